// moe.hip -- MoE FFN block with a fixed routing-order combine, for gfx950.
//
// "IsoExec: Eliminating Trainer-Inference Mismatch in SkyRL" (agentlenshq),
// section "Achieving Parallelism Invariance", EP bullet, and the
// katelyatop-blog post on vLLM/SkyRL IsoExec, section 9: expert outputs are
// combined in a fixed routing order, not in the order ranks (or, on one GPU,
// workgroups) finish.  Every step below computes a token's numbers from that
// token's own data with a fixed order, so a token's output bits do not depend
// on the other tokens in the batch or on their order:
//   route    one wave per token: softmax over the expert logits (max, exp,
//            balanced tree over expert index), top_k by (logit descending,
//            expert id ascending) = the routing order, gates renormalised by
//            a balanced tree over the selected probabilities;
//   bucket   per expert, the (token, slot) pairs that chose it, in token
//            order (order-preserving compaction, no atomics);
//   plan     the list of (expert, 128-row tile) work items;
//   experts  grouped leaf/tree GEMMs over the gathered rows: G = x Wg[e] and
//            U = x Wu[e] with h = bf16(silu(G) U) fused, then out = h Wd[e];
//   combine  y = g_0 out_0, then y += g_k out_k for k = 1..top_k-1 (each
//            product rounded before its add).
#include <type_traits>

#include "gemm_core.hpp"
#include "gemm_wide.hpp"
#include "kernels.h"

namespace iso {

// ------------------------------------------------------------------ route

// Balanced tree over the 64 lanes of a wave in lane order; every lane ends
// with the root.  Inside each row of 16 lanes the levels pair lanes l ^ 1,
// l ^ 2, then the other quad of the 8 and the other 8 of the 16 (DPP, the
// same sums as l ^ 4 and l ^ 8 since IEEE addition is commutative), then
// rows l ^ 16 and l ^ 32.
__device__ __forceinline__ float wave_tree_sum(float v)
{
    v = row16_sum(v);
    v = v + shfl_xor(v, 16);
    return v + shfl_xor(v, 32);
}

template <int CTRL>
__device__ __forceinline__ int dpp_int(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}

// The wave's largest (value, -expert) pair: a total order, so any pairing of
// lanes gives the same winner; DPP inside rows of 16, then l ^ 16 and l ^ 32.
// NaN values never win.
__device__ __forceinline__ void wave_argmax(float &bv, int &be)
{
    auto take = [&](float ov, int oe) {
        if (ov > bv || (ov == bv && oe < be)) {
            bv = ov;
            be = oe;
        }
    };
    take(dpp_mov<0xB1>(bv), dpp_int<0xB1>(be));
    take(dpp_mov<0x4E>(bv), dpp_int<0x4E>(be));
    take(dpp_mov<0x141>(bv), dpp_int<0x141>(be));
    take(dpp_mov<0x140>(bv), dpp_int<0x140>(be));
    take(shfl_xor(bv, 16), __shfl_xor(be, 16, 64));
    take(shfl_xor(bv, 32), __shfl_xor(be, 32, 64));
}

// Balanced tree over n = 2^k register values in index order.
template <int N>
__device__ __forceinline__ float reg_tree_sum(float (&v)[N])
{
#pragma unroll
    for (int width = N; width > 1; width >>= 1)
#pragma unroll
        for (int q = 0; q < width / 2; ++q)
            v[q] = v[2 * q] + v[2 * q + 1];
    return v[0];
}

constexpr int kMaxTopK = 16;

// Lane l holds experts e = 64 q + l, q < Q (Q * 64 >= E, Q a power of two).
template <int Q>
__global__ __launch_bounds__(256) void moe_route_kernel(const float *logits, int32_t *idx,
                                                        float *gate, int64_t T, int E, int top_k)
{
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= T)
        return;
    const float *l = logits + t * E;
    float lg[Q];
    bool taken[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int e = q * 64 + lane;
        lg[q] = e < E ? l[e] : -INFINITY;
        taken[q] = e >= E;
    }
    float mx = lg[0];
#pragma unroll
    for (int q = 1; q < Q; ++q)
        mx = fmaxf(mx, lg[q]);
    mx = row16_max(mx);  // max is exact in any order
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));

    float p[Q], blk[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        p[q] = (q * 64 + lane) < E ? exp_neg(lg[q] - mx) : 0.0f;
        blk[q] = wave_tree_sum(p[q]);  // 64-expert blocks, aligned subtrees
    }
    const float z = reg_tree_sum(blk);

    // top_k in routing order; probabilities of the chosen experts
    float psel[kMaxTopK];
    int esel[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        psel[k] = 0.0f;
        esel[k] = 0;
        if (k >= top_k)
            continue;
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int e = q * 64 + lane;
            if (!taken[q] && (lg[q] > bv || (lg[q] == bv && e < be))) {
                bv = lg[q];
                be = e;
            }
        }
        wave_argmax(bv, be);
        // expert be sits in lane be & 63, register q = be >> 6 (the same on all lanes)
        float pv = 0.0f;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if (q * 64 + lane == be)
                taken[q] = true;
            if (q == (be >> 6))
                pv = __shfl(p[q], be & 63, 64);
        }
        psel[k] = pv / z;
        esel[k] = be;
    }
    // renormalise over the selected ones: balanced tree in routing order
    // (slots past top_k hold +0.0, which leaves every partial sum unchanged)
    float s[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        s[k] = psel[k];
    const float ssum = reg_tree_sum(s);
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k == lane && k < top_k) {
            idx[t * top_k + k] = esel[k];
            gate[t * top_k + k] = psel[k] / ssum;
        }
}

// --------------------------------------------------------------- bucket

// Expert e = blockIdx.x gathers the entries i = t * top_k + slot with
// idx[i] == e, in increasing i, into rows[e][0 .. count).  The entries go
// through LDS in chunks of 32768 (direct global-to-LDS loads, all in flight
// together).  In a chunk, wave w scans the contiguous quarter w, 64 entries
// at a time; a ballot ranks each match among the wave's matches (lanes below
// it).  A first pass counts the matches of every quarter, so that quarter w
// starts after the matches of quarters 0 .. w-1; the second pass writes.
constexpr int kBucketChunk = 32768;

__global__ __launch_bounds__(256) void moe_bucket_kernel(const int32_t *idx, int32_t *rows,
                                                         int32_t *counts, int64_t n_entries,
                                                         int64_t T)
{
    __shared__ __attribute__((aligned(16))) int32_t sidx[kBucketChunk];
    __shared__ int wcount[4];
    const int e = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t below = (1ull << lane) - 1;
    int32_t *dst = rows + static_cast<int64_t>(e) * T;
    int count = 0;
    for (int64_t base = 0; base < n_entries; base += kBucketChunk) {
        const int n = n_entries - base < kBucketChunk ? static_cast<int>(n_entries - base)
                                                       : kBucketChunk;
        // 128 KiB: each wave loads 32 KiB, 1 KiB per instruction; entries
        // past n read as 0 and are never scanned
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t *>(idx + base), (short)0, n * 4, 0x00020000);
#pragma unroll
        for (int j = 0; j < kBucketChunk / 1024; ++j) {
            const int off = w * kBucketChunk + j * 1024;  // bytes: wave w's 32 KiB, then 1 KiB steps
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (ISO_LDS void *)(reinterpret_cast<char *>(sidx) + off), 16,
                static_cast<uint32_t>(lane * 16), static_cast<uint32_t>(off), 0, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        const int q = ((n + 255) / 256) * 64;  // entries per quarter, a multiple of 64
        const int lo = w * q;
        const int hi = lo + q < n ? lo + q : n;
        constexpr int U = 8;  // independent LDS reads per step
        int c = 0;
        for (int i0 = lo; i0 < hi; i0 += 64 * U) {
            bool m[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + 64 * u + lane;
                m[u] = i < hi && sidx[i < kBucketChunk ? i : 0] == e;
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                c += __popcll(__ballot(m[u]));
        }
        if (lane == 0)
            wcount[w] = c;
        __syncthreads();
        int pos = count;
        for (int k = 0; k < w; ++k)
            pos += wcount[k];
        for (int i0 = lo; i0 < hi; i0 += 64 * U) {
            bool m[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = i0 + 64 * u + lane;
                m[u] = i < hi && sidx[i < kBucketChunk ? i : 0] == e;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint64_t mask = __ballot(m[u]);
                if (m[u])
                    dst[pos + __popcll(mask & below)] =
                        static_cast<int32_t>(base + i0 + 64 * u + lane);
                pos += __popcll(mask);
            }
        }
        count += (wcount[0] + wcount[1]) + (wcount[2] + wcount[3]);
        __syncthreads();  // the next chunk overwrites sidx and wcount
    }
    if (threadIdx.x == 0)
        counts[e] = count;
}

// Two-pass bucket (T <= kMoeBucketMaxT): the same lists, built from blocks of
// 64 tokens.  A token's top_k experts are distinct, so in a block expert e
// takes at most one entry per token, and an entry's place among the block's
// entries of e is the number of earlier tokens of the block that chose e:
// the population count of a 64-bit token mask below the token.  Counts and
// masks are built with LDS atomics, whose results do not depend on their
// order; entries land at the expert's count over the earlier blocks plus
// that place, i.e. in token order.  Entries with an expert id outside
// [0, E) (a token whose logits were all NaN) belong to no expert.
__global__ __launch_bounds__(1024) void moe_bucket_count_kernel(const int32_t *idx, int32_t *blk,
                                                                int64_t T, int E, int top_k)
{
    __shared__ int c_s[1024];
    const int64_t b = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        c_s[e] = 0;
    __syncthreads();
    const int64_t t0 = b * kMoeBucketTok;
    const int nt = T - t0 < kMoeBucketTok ? static_cast<int>(T - t0) : kMoeBucketTok;
    for (int j = threadIdx.x; j < nt * top_k; j += blockDim.x) {
        const int e = idx[t0 * top_k + j];
        if (e >= 0 && e < E)
            atomicAdd(&c_s[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        blk[b * E + e] = c_s[e];
}

__global__ __launch_bounds__(1024) void moe_bucket_scatter_kernel(const int32_t *idx,
                                                                  const int32_t *blk,
                                                                  int32_t *rows, int32_t *counts,
                                                                  int64_t T, int E, int top_k)
{
    __shared__ int base_s[1024];
    __shared__ int part_s[1024];
    __shared__ unsigned long long mask_s[1024];
    const int64_t b = blockIdx.x;
    const int64_t nb = gridDim.x;
    // the expert's count over the earlier blocks: parts threads per expert
    // each sum every parts-th block (integers: the order does not matter)
    const int parts = static_cast<int>(blockDim.x) / E;
    if (static_cast<int>(threadIdx.x) < parts * E) {
        const int e = threadIdx.x % E, part = threadIdx.x / E;
        int s = 0;
#pragma unroll 4
        for (int64_t q = part; q < b; q += parts)
            s += blk[q * E + e];
        part_s[part * E + e] = s;
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        mask_s[e] = 0ull;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int s = 0;
        for (int part = 0; part < parts; ++part)
            s += part_s[part * E + e];
        base_s[e] = s;
        if (b == nb - 1)
            counts[e] = s + blk[b * E + e];
    }
    __syncthreads();
    const int64_t t0 = b * kMoeBucketTok;
    const int nt = T - t0 < kMoeBucketTok ? static_cast<int>(T - t0) : kMoeBucketTok;
    for (int j = threadIdx.x; j < nt * top_k; j += blockDim.x) {
        const int e = idx[t0 * top_k + j];
        if (e >= 0 && e < E)
            atomicOr(&mask_s[e], 1ull << (j / top_k));
    }
    __syncthreads();
    for (int j = threadIdx.x; j < nt * top_k; j += blockDim.x) {
        const int e = idx[t0 * top_k + j];
        if (e >= 0 && e < E) {
            const int tl = j / top_k;
            const int place = __popcll(mask_s[e] & ((1ull << tl) - 1ull));
            rows[static_cast<int64_t>(e) * T + base_s[e] + place] =
                static_cast<int32_t>(t0 * top_k + j);
        }
    }
}

// ------------------------------------------------------------------ plan

// Work list of 128-row tiles in expert order, each (expert, first row, the
// expert's first tile, its tile count): thread e (E <= 1024 threads) scans
// the per-expert tile counts and writes its own tiles.
__global__ __launch_bounds__(1024) void moe_plan_kernel(const int32_t *counts, int32_t *tiles,
                                                        int32_t *ntiles, int E)
{
    __shared__ int scan[1024];
    const int e = threadIdx.x;
    const int c = e < E ? counts[e] : 0;
    const int mine = (c + BM - 1) / BM;
    scan[e] = mine;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int add = e >= d ? scan[e - d] : 0;
        __syncthreads();
        scan[e] += add;
        __syncthreads();
    }
    const int first = scan[e] - mine;
    int n = first;
    for (int m0 = 0; m0 < c; m0 += BM, ++n) {
        tiles[4 * n] = e;
        tiles[4 * n + 1] = m0;
        tiles[4 * n + 2] = first;
        tiles[4 * n + 3] = mine;
    }
    if (e == 1023)
        *ntiles = scan[1023];
}

// --------------------------------------------------------------- experts

struct MoeGemmArgs {
    const uint16_t *A;       // gathered operand: X [T][H] or h [T*k][I]
    int64_t a_rows_total;    // rows of A (for the range check)
    int row_div;             // source row = entry / row_div (top_k for X, 1 for h)
    const uint16_t *B0;      // Wg or Wd  [E][N][K]
    const uint16_t *B1;      // Wu (gate/up only)
    void *out;               // h [T*k][N] bf16 or e [T*k][N] fp32
    const int32_t *rows;     // [E][T]
    const int32_t *counts;   // [E]
    const int32_t *tiles;    // [ntiles][2]
    const int32_t *ntiles;   // [1]
    int64_t T, N, K;
    int stages_per_leaf;
};

// One work item: an expert's 128-row tile (rows m0 .. m0+nvalid-1 of its
// bucket) times output columns n0 .. n0+TN-1.
struct MoeTask {
    int e, m0, nvalid;
    int64_t n0;
};

__device__ __forceinline__ MoeTask moe_task(const int32_t *__restrict__ tiles,
                                            const int32_t *__restrict__ counts, int w, int ntn,
                                            int tn_cols)
{
    MoeTask t;
    // an expert's tasks are contiguous, row tiles fastest: the tasks that
    // share a weight column tile run next to each other (one L2)
    const int q = w / ntn;
    const int first = __builtin_amdgcn_readfirstlane(tiles[4 * q + 2]);
    const int ntl = __builtin_amdgcn_readfirstlane(tiles[4 * q + 3]);
    const int local = w - first * ntn;
    const int tile = first + local % ntl;
    t.n0 = static_cast<int64_t>(local / ntl) * tn_cols;
    t.e = __builtin_amdgcn_readfirstlane(tiles[4 * tile]);
    t.m0 = __builtin_amdgcn_readfirstlane(tiles[4 * tile + 1]);
    const int cnt = __builtin_amdgcn_readfirstlane(counts[t.e]);
    t.nvalid = cnt - t.m0 < BM ? cnt - t.m0 : BM;
    return t;
}

// The task's bucket entries rows[e][m0 .. m0+127] into dst (LDS) by direct
// global-to-LDS loads of the first two waves; entries past the bucket read
// as 0 and are never used.  Tracked by the vector memory counter.
__device__ __forceinline__ void rows_dma(const MoeGemmArgs &a, const MoeTask &t, int32_t *dst)
{
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w < BM / 64) {
        const int32_t *src = a.rows + static_cast<int64_t>(t.e) * a.T + t.m0;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t *>(src), (short)0, t.nvalid * 4, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ISO_LDS void *)(dst + 64 * w), 4,
                                                 static_cast<uint32_t>(lane_id() * 4),
                                                 static_cast<uint32_t>(w * 256), 0, 0);
    }
}

// Gate/up tiles hold 64 intermediate columns: B rows 0..63 of the tile are
// Wg rows n0..n0+63 (loaded by the first half of the waves) and B rows
// 64..127 are the same Wu rows (second half), so one contraction yields G in
// tile columns 0..63 and U in columns 64..127 of every row.
constexpr int kGuCols = BN / 2;

// Pipe over gathered A rows: DMA row r of the tile reads source row
// rows_s[r] / row_div of the whole A matrix, or zero when r >= nvalid (its
// offset lies past the buffer's range).  rows_s: the task's entries in LDS.
template <class C, bool GATE_UP>
__device__ __forceinline__ Pipe moe_pipe(const MoeGemmArgs &a, const MoeTask &t,
                                         const int32_t *rows_s)
{
    const int64_t boff = static_cast<int64_t>(t.e) * a.N * a.K + t.n0 * a.K;
    Pipe p = make_pipe<C>(a.A, 0, a.B0 + boff, a.N - t.n0, a.K, 0);
    p.ra = tile_rsrc(a.A, a.a_rows_total, a.K);
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t c = (lane & 7) ^ (lane >> 3);
    const uint32_t oob = (uint32_t)(a.a_rows_total * a.K * 2);
    int32_t ent[C::kDma];
#pragma unroll
    for (int i = 0; i < C::kDma; ++i)
        lds_issue_b32(ent[i], lds_addr(rows_s + C::kDma * 8 * w + 8 * i + (lane >> 3)));
    lds_wait();
    // re-read for every task (see moe_gu_pipe_w)
    int row_div = a.row_div;
    asm volatile("" : "+s"(row_div));
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) {
        lds_pin(ent[i]);
        const int r = C::kDma * 8 * w + 8 * i + (lane >> 3);
        if (r < t.nvalid) {
            const int64_t src = ent[i] / row_div;
            p.voffa[i] = (uint32_t)(src * a.K * 2) + c * 16;
        } else {
            p.voffa[i] = oob;
        }
    }
    if constexpr (GATE_UP) {
        const int64_t brows = a.N - t.n0 < kGuCols ? a.N - t.n0 : kGuCols;
        p.rb = tile_rsrc((w < C::kWaves / 2 ? a.B0 : a.B1) + boff, brows, a.K);
#pragma unroll
        for (int i = 0; i < C::kDma; ++i) {
            const uint32_t r = (C::kDma * 8 * w + 8 * i + (lane >> 3)) & (kGuCols - 1);
            p.voffb[i] = (uint32_t)((int64_t)r * a.K * 2) + c * 16;
        }
    }
    return p;
}

// Rows 64h .. 64h+63 of a tile's roots (held by the waves of tile row h) into
// `stg` [64][128] FP32, with the chunk swizzle of stage_tile.
template <class C>
__device__ __forceinline__ void stage_half(const Acc<C> &root, float *stg, int h)
{
    static_assert(C::WR == 2 && BM == 128, "two wave rows of 64 tile rows");
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / C::WC, wc = wave % C::WC;
    if (wr != h)
        return;
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
#pragma unroll
        for (int j = 0; j < C::JB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = tile_row<C>(lane, wr, i, r) - 64 * h;
                const int col = tile_col<C>(lane, wc, j);
                const int chunk = (col >> 2) ^ (((row >> 2) & 3) << 2);
                lds_write_f32(lds_addr(stg + row * 128 + chunk * 4 + (col & 3)), root.v[i][j][r]);
            }
}

// Columns 4c .. 4c+3 of row `row` of a [64][128] staging buffer (address).
__device__ __forceinline__ uint32_t staged_addr(const float *stg, int row, int c)
{
    return lds_addr(stg + row * 128 + ((c ^ (((row >> 2) & 3) << 2)) << 2));
}

// Epilogue of one task: gate/up writes h = bf16(silu(G) U) (G in tile
// columns 0..63, U in 64..127), down writes the FP32 roots; tile row r goes
// to output row rows_s[r].  Two halves of 64 rows through `stg` (32 KiB).
template <class C, bool GATE_UP>
__device__ __forceinline__ void moe_epilogue(const MoeGemmArgs &a, const MoeTask &t,
                                             const Acc<C> &r0, const int32_t *rows_s, float *stg)
{
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
        stage_half<C>(r0, stg, h);
        lds_barrier();
        if constexpr (GATE_UP) {
            constexpr int UPT = 64 * (kGuCols / 8) / C::kThreads;  // units per thread
            uint16_t *o = static_cast<uint16_t *>(a.out) + t.n0;
            const bool al = (reinterpret_cast<uintptr_t>(o) % 16 == 0) && (a.N % 8 == 0);
            const int cmax = a.N - t.n0 < kGuCols ? static_cast<int>(a.N - t.n0) : kGuCols;
            constexpr int NB = UPT < 2 ? UPT : 2;  // units per LDS round trip
#pragma unroll
            for (int kb = 0; kb < UPT; kb += NB) {
            f32x4 g0[NB], g1[NB], u0[NB], u1[NB];
            int32_t dst[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int u = threadIdx.x + (kb + k) * C::kThreads;
                const int row = u >> 3, q = u & 7;
                lds_issue_b128(g0[k], staged_addr(stg, row, 2 * q));
                lds_issue_b128(g1[k], staged_addr(stg, row, 2 * q + 1));
                lds_issue_b128(u0[k], staged_addr(stg, row, kGuCols / 4 + 2 * q));
                lds_issue_b128(u1[k], staged_addr(stg, row, kGuCols / 4 + 2 * q + 1));
                lds_issue_b32(dst[k], lds_addr(rows_s + 64 * h + row));
            }
            lds_wait();
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                lds_pin(g0[k]);
                lds_pin(g1[k]);
                lds_pin(u0[k]);
                lds_pin(u1[k]);
                lds_pin(dst[k]);
                const int u = threadIdx.x + (kb + k) * C::kThreads;
                const int row = u >> 3, q = u & 7;
                if (64 * h + row >= t.nvalid)
                    continue;
                const float gs[8] = {g0[k][0], g0[k][1], g0[k][2], g0[k][3],
                                     g1[k][0], g1[k][1], g1[k][2], g1[k][3]};
                const float us[8] = {u0[k][0], u0[k][1], u0[k][2], u0[k][3],
                                     u1[k][0], u1[k][1], u1[k][2], u1[k][3]};
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = swiglu_act(gs[e], us[e]);
                store8_bf16(o + static_cast<int64_t>(dst[k]) * a.N + 8 * q, v,
                            al && 8 * q + 8 <= cmax, cmax - 8 * q);
            }
            }
        } else {
            constexpr int UPT = 64 * 32 / C::kThreads;  // units per thread
            float *o = static_cast<float *>(a.out) + t.n0;
            const bool al = (reinterpret_cast<uintptr_t>(o) % 16 == 0) && (a.N % 4 == 0);
            const int cmax = a.N - t.n0 < BN ? static_cast<int>(a.N - t.n0) : BN;
            constexpr int NB = UPT < 4 ? UPT : 4;  // units per LDS round trip
#pragma unroll
            for (int kb = 0; kb < UPT; kb += NB) {
            f32x4 v[NB];
            int32_t dst[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int u = threadIdx.x + (kb + k) * C::kThreads;
                const int row = u >> 5, q = u & 31;
                lds_issue_b128(v[k], staged_addr(stg, row, q));
                lds_issue_b32(dst[k], lds_addr(rows_s + 64 * h + row));
            }
            lds_wait();
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                lds_pin(v[k]);
                lds_pin(dst[k]);
                const int u = threadIdx.x + (kb + k) * C::kThreads;
                const int row = u >> 5, q = u & 31;
                if (64 * h + row >= t.nvalid)
                    continue;
                store4_f32(o + static_cast<int64_t>(dst[k]) * a.N + 4 * q, v[k],
                           al && 4 * q + 4 <= cmax, cmax - 4 * q);
            }
            }
        }
        lds_barrier();
    }
}

// Persistent over the task list.  XCD-aware split: the workgroups on XCD x
// (blockIdx % 8 == x) take the contiguous task range [x per, (x+1) per), so
// the tasks running together on one L2 share an expert's weights and a
// tile's rows; the grid is a multiple of 8, so every task is taken once.
//
// OVERLAP (eight-wave shape, three-stage ring): the next task's bucket
// entries are fetched during the current main loop, and its first ring
// stages are requested right after it, before the epilogue, which stages
// through its own LDS.  Otherwise (four-wave shape, two workgroups per CU)
// each task runs start to end and the epilogue stages through the ring.
template <class C, int LOG, bool GATE_UP>
__global__ __launch_bounds__(C::kThreads, 2) void moe_expert_kernel(
    MoeGemmArgs a, const int32_t *__restrict__ tiles, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ ntiles)
{
    constexpr bool OVERLAP = C::kWaves == 8;
    __shared__ __attribute__((aligned(16))) char lds[C::kLdsBytes];
    __shared__ __attribute__((aligned(16))) float stg_own[OVERLAP ? 64 * 128 : 4];
    __shared__ int32_t rows_s[2][BM];
    static_assert(OVERLAP || C::kLdsBytes >= 64 * 128 * 4, "the ring must hold half a tile");
    float *stg = OVERLAP ? stg_own : reinterpret_cast<float *>(lds);

    constexpr int TN = GATE_UP ? kGuCols : BN;  // output columns per tile
    const int ntn = static_cast<int>((a.N + TN - 1) / TN);
    const int total = __builtin_amdgcn_readfirstlane(*ntiles) * ntn;
    const int xcd = blockIdx.x % kXcds;
    const int slots = gridDim.x / kXcds;
    const int per = (total + kXcds - 1) / kXcds;
    const int end = (xcd + 1) * per < total ? (xcd + 1) * per : total;
    int w = xcd * per + static_cast<int>(blockIdx.x) / kXcds;
    if (w >= end)
        return;
    const int nst = (1 << LOG) * a.stages_per_leaf;

    {
        const MoeTask t = moe_task(tiles, counts, w, ntn, TN);
        rows_dma(a, t, rows_s[0]);
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if constexpr (OVERLAP)
            pipe_prologue<C>(moe_pipe<C, GATE_UP>(a, t, rows_s[0]), lds, nst);
    }
    for (int it = 0;; ++it) {
        const int b = it & 1;
        const MoeTask t = moe_task(tiles, counts, w, ntn, TN);
        const int wn = w + slots;
        Acc<C> r0;
        // re-read per task (see moe_gu_wide_kernel)
        int spl = a.stages_per_leaf;
        asm volatile("" : "+s"(spl));
        if constexpr (OVERLAP) {
            const Pipe p = moe_pipe<C, GATE_UP>(a, t, rows_s[b]);
            if (wn < end)
                rows_dma(a, moe_task(tiles, counts, wn, ntn, TN), rows_s[b ^ 1]);
            leaf_tree_mainloop<C, LOG, false>(p, spl, lds, r0);
            if (wn < end)
                pipe_prologue<C>(moe_pipe<C, GATE_UP>(a, moe_task(tiles, counts, wn, ntn, TN), rows_s[b ^ 1]),
                                 lds, nst);
        } else {
            leaf_tree_mainloop<C, LOG>(moe_pipe<C, GATE_UP>(a, t, rows_s[b]), spl, lds, r0);
            if (wn < end)
                rows_dma(a, moe_task(tiles, counts, wn, ntn, TN), rows_s[b ^ 1]);
        }
        moe_epilogue<C, GATE_UP>(a, t, r0, rows_s[b], stg);
        if (wn >= end)
            break;
        if constexpr (!OVERLAP)
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // next entries landed
        w = wn;
    }
}

// ------------------------------------------- gate/up on 128 x 256 tiles

// A wide gate/up task covers 128 intermediate columns n0 .. n0+127.  Its B
// rows are 16-row blocks that alternate between Wg and Wu: block 2k holds Wg
// rows n0 + 16k .. n0 + 16k + 15 and block 2k+1 the same Wu rows.  Wave
// column wc then holds G in its column blocks 2k and U in blocks 2k+1 for
// the same intermediate columns n0 + 16 (4 wc + k) .. + 15, element for
// element in matching registers, and h = bf16(silu(G) U) is formed in
// registers (the same device function as every other SwiGLU here).
constexpr int kGuColsW = 128;

// Ring loads of a wide gate/up task: A rows gathered as in moe_pipe; B group
// i of wave w is block 4 w + (i >> 1), i.e. Wg for (i & 2) == 0, else Wu.
__device__ __forceinline__ PipeW moe_gu_pipe_w(const MoeGemmArgs &a, const MoeTask &t,
                                               const int32_t *rows_s)
{
    PipeW p;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t c = (lane & 7) ^ (lane >> 3);
    p.ra = tile_rsrc(a.A, a.a_rows_total, a.K);
    const uint32_t oob = (uint32_t)(a.a_rows_total * a.K * 2);
    int32_t ent[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        lds_issue_b32(ent[i], lds_addr(rows_s + 32 * w + 8 * i + (lane >> 3)));
    lds_wait();
    // the divisor as a value the compiler re-reads for every task: its
    // reciprocal would otherwise be hoisted out of the task loop and spilled,
    // and the reload waits for every memory operation, the previous task's
    // stores included
    int row_div = a.row_div;
    asm volatile("" : "+s"(row_div));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lds_pin(ent[i]);
        const int r = 32 * w + 8 * i + (lane >> 3);
        p.voffa[i] = r < t.nvalid ? (uint32_t)((int64_t)(ent[i] / row_div) * a.K * 2) + c * 16
                                  : oob;
    }
    const int64_t boff = static_cast<int64_t>(t.e) * a.N * a.K + t.n0 * a.K;
    const int64_t brows = a.N - t.n0 < kGuColsW ? a.N - t.n0 : kGuColsW;
    p.rb = tile_rsrc(a.B0 + boff, brows, a.K);
    p.rb2 = tile_rsrc(a.B1 + boff, brows, a.K);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t r = (uint32_t)((((4 * w + (i >> 1)) >> 1) << 4) + 8 * (i & 1) + (lane >> 3));
        p.voffb[i] = (uint32_t)((int64_t)r * a.K * 2) + c * 16;
    }
    p.kbyte0 = 0;
    return p;
}

// h of a wide task straight from the transposed accumulators (no staging):
// lane l of wave (wr, wc) holds, for row block i, G (block 2k) and U (block
// 2k + 1) of the four h columns 16 (4 wc + k) + 4 (l >> 4) + q of row 64 wr
// + 16 i + (l & 15), which leave as one 8-byte store.
__device__ __forceinline__ void moe_gu_epilogue_t(const MoeGemmArgs &a, const MoeTask &t,
                                                  const AccW &r, const int32_t *rows_s)
{
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave >> 1, wc = wave & 1;
    // the four bucket entries of this lane's rows, read and waited for in
    // one asm statement (an output of an LDS read left in flight across
    // statements may be copied before it has arrived)
    int32_t dst[4];
    {
        const uint32_t e0 = lds_addr(rows_s + wr * 64 + (lane & 15));
        asm volatile("ds_read_b32 %0, %4\n\t"
                     "ds_read_b32 %1, %4 offset:64\n\t"
                     "ds_read_b32 %2, %4 offset:128\n\t"
                     "ds_read_b32 %3, %4 offset:192\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(dst[0]), "=&v"(dst[1]), "=&v"(dst[2]), "=&v"(dst[3])
                     : "v"(e0)
                     : "memory");
    }
    int64_t hbytes = a.a_rows_total * a.row_div * a.N * 2;
    if (hbytes > 0xffffffffLL)
        hbytes = 0xffffffffLL;
    const __amdgpu_buffer_rsrc_t hr =
        __builtin_amdgcn_make_buffer_rsrc(a.out, (short)0, (int)(uint32_t)hbytes, 0x00020000);
    const bool al = (reinterpret_cast<uintptr_t>(a.out) % 8 == 0) && (a.N % 4 == 0) &&
                    (t.n0 % 4 == 0);
    const int cmax = a.N - t.n0 < kGuColsW ? static_cast<int>(a.N - t.n0) : kGuColsW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (wr * 64 + i * 16 + (lane & 15) >= t.nvalid)
            continue;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t hv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                hv[q] = f32_to_bf16_rne(swiglu_act(r.v[i][2 * k][q], r.v[i][2 * k + 1][q]));
            const int col = (4 * wc + k) * 16 + 4 * (lane >> 4);
            const uint32_t off = (uint32_t)((dst[i] * a.N + t.n0 + col) * 2);
            if (al && col + 4 <= cmax) {
                u32x2 v;
                v[0] = hv[0] | (hv[1] << 16);
                v[1] = hv[2] | (hv[3] << 16);
                __builtin_amdgcn_raw_buffer_store_b64(v, hr, off, 0, 0);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (col + q < cmax)
                        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(hv[q]), hr,
                                                              off + 2 * q, 0, 0);
            }
        }
    }
    // the next task's bucket entries go into the other half of rows_s only
    // after every wave has read this half
    __builtin_amdgcn_s_barrier();
}

// Persistent over the wide gate/up tasks, one workgroup per CU, with the
// XCD-aware task split of moe_expert_kernel.  The next task's bucket entries
// are fetched during the main loop; the MFMAs take the weights as their
// first operand, so the epilogue stores h straight from registers.
// (Requesting the next task's first ring stages before the epilogue measured
// no faster, and a register reload in the epilogue would then wait for those
// loads.)
template <int LOG>
__global__ __launch_bounds__(256, 1) void moe_gu_wide_kernel(MoeGemmArgs a,
                                                             const int32_t *__restrict__ tiles,
                                                             const int32_t *__restrict__ counts,
                                                             const int32_t *__restrict__ ntiles)
{
    __shared__ __attribute__((aligned(16))) char lds[kWLdsBytes];
    __shared__ int32_t rows_s[2][BM];
    const int ntn = static_cast<int>((a.N + kGuColsW - 1) / kGuColsW);
    const int total = __builtin_amdgcn_readfirstlane(*ntiles) * ntn;
    const int xcd = blockIdx.x % kXcds;
    const int slots = gridDim.x / kXcds;
    const int per = (total + kXcds - 1) / kXcds;
    const int end = (xcd + 1) * per < total ? (xcd + 1) * per : total;
    int w = xcd * per + static_cast<int>(blockIdx.x) / kXcds;
    if (w >= end)
        return;
    rows_dma(a, moe_task(tiles, counts, w, ntn, kGuColsW), rows_s[0]);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    for (int it = 0;; ++it) {
        const int b = it & 1;
        const MoeTask t = moe_task(tiles, counts, w, ntn, kGuColsW);
        const int wn = w + slots;
        const PipeW p = moe_gu_pipe_w(a, t, rows_s[b]);
        if (wn < end)
            rows_dma(a, moe_task(tiles, counts, wn, ntn, kGuColsW), rows_s[b ^ 1]);
        AccW r0;
        // stages per leaf as a value the compiler re-reads for every task:
        // conditions derived from it would otherwise be hoisted out of the
        // task loop and spilled, and their reload waits for every load
        int spl = a.stages_per_leaf;
        asm volatile("" : "+s"(spl));
        leaf_tree_mainloop_w<LOG, true>(p, spl, lds, r0);
        moe_gu_epilogue_t(a, t, r0, rows_s[b]);
        if (wn >= end)
            break;
        w = wn;
    }
}

// ------------------------------- down projection with the rows in registers

// A down task: an expert's 128-row tile times up to kDnCT column tiles of
// 128 output columns.  Each of the four waves (one per SIMD) holds 32 of the
// task's rows of h (K = I = 32 KS) in AGPRs, for all the task's column
// tiles (each wave loads only its own rows); the Wd rows stream through a
// ring of four 16 KiB LDS stages (128 rows x 64 k, chunk-swizzled as in
// gemm_core.hpp), one column tile after another without draining; every
// wave reads all 128 columns of each stage.  The MFMA takes the weights as
// its first operand and the rows as its second: every output element is
// still the same products summed in the same k order from +0.0 (the same
// leaves and tree as every other kernel), and a lane's four accumulator
// values are four consecutive output columns of one row, which leave as one
// 16-byte store straight from registers.
constexpr int kDnCT = 4;
constexpr int kDnStage = 128 * kRowBytes;  // 16 KiB
constexpr int kDnBuf = 4;

template <int KS>
struct DnRows {
    bf16x8 v[2][KS];  // row block i (16 rows), k-step
};
struct DnAcc {
    f32x4 v[2][8];  // row block i, column block j
};
struct DnFrags {
    bf16x8 b[8];  // column blocks of one k-step
};

// acc (+)= Wd block x rows block (the transposed product; see above).
template <bool FRESH>
__device__ __forceinline__ void mfma_dn(f32x4 &acc, const bf16x8 &w, const bf16x8 &r)
{
    if constexpr (FRESH)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(w), "a"(r));
    else
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(w), "a"(r));
}

template <int J>
__device__ __forceinline__ void dn_frag(DnFrags &f, uint32_t addr)
{
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(f.b[J]) : "v"(addr), "i"(J * 16 * kRowBytes));
}

__device__ __forceinline__ void dn_frags_wait(DnFrags &f)
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < 8; ++j)
        asm volatile("" : "+v"(f.b[j]));
}

// Ring load q of global stage g of the task (column tile g / spt, k stage
// g % spt) for this wave: Wd rows 32 w + 8 q + (lane >> 3) of the tile.
__device__ __forceinline__ void dn_dma(__amdgpu_buffer_rsrc_t rb, const uint32_t (&voff)[4],
                                       char *lds, int g, int spt, int64_t K, int q)
{
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = g / spt, st = g - c * spt;
    const uint32_t soff = (uint32_t)(c * 128 * K * 2) + (uint32_t)st * (BK * 2);
    char *dst = lds + (g % kDnBuf) * kDnStage + (w * 32 + q * 8) * kRowBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (ISO_LDS void *)dst, 16, voff[q], soff, 0, 0);
}

// Rows of a task: this lane's 16-byte piece of k-step ks of row block i
// (row 32 w + 16 i + (lane & 15), k 32 ks + 8 (lane >> 4) ..), read through
// `ra` at byte offset base[i] + 64 ks (past the range: zeros).
template <int KS>
__device__ __forceinline__ void dn_row_load(DnRows<KS> &rows, __amdgpu_buffer_rsrc_t ra,
                                            const uint32_t (&base)[2], int i, int ks)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ra, base[i] + ks * 64, 0, 0);
    rows.v[i][ks] = reinterpret_cast<const bf16x8 &>(v);
}

// s_waitcnt vmcnt(n) for n in {0, 4, 8, 12}, then a workgroup barrier.
// Later stores only make the wait stricter.
__device__ __forceinline__ void dn_vm_barrier(int n)
{
    switch (n) {
    case 12: asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); break;
    }
}

__device__ __forceinline__ void dn_drain(DnAcc &acc)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            asm volatile("" : "+v"(acc.v[i][j]));
}

// Tree level 1 (the sum of two leaves, saved while the next two run) of a
// four-leaf tree is kept in LDS, each wave in its own 16 KiB (three register
// sets of 64 do not fit beside the rows and fragments); the values pass
// unchanged.  `l1` is this lane's address in that region.
__device__ __forceinline__ void dn_park_lds(const DnAcc &v, uint32_t l1)
{
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(l1), "v"(v.v[i][j]),
                         "i"((i * 8 + j) * 1024)
                         : "memory");
}

__device__ __forceinline__ void dn_unpark_lds(DnAcc &left, uint32_t l1)
{
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            asm volatile("ds_read_b128 %0, %1 offset:%2"
                         : "=v"(left.v[i][j])
                         : "v"(l1), "i"((i * 8 + j) * 1024));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            asm volatile("" : "+v"(left.v[i][j]));
}

template <int LOG, int J, int B>
__device__ __forceinline__ void dn_tree_push(DnAcc (&stk)[LOG > 0 ? LOG : 1], DnAcc &v, uint32_t l1)
{
    constexpr bool IN_LDS = LOG == 2 && B == 1;
    if constexpr (B < LOG) {
        if constexpr (((J >> B) & 1) != 0) {
            if constexpr (IN_LDS)
                dn_unpark_lds(stk[B], l1);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v.v[i][j] = stk[B].v[i][j] + v.v[i][j];
            dn_tree_push<LOG, J, B + 1>(stk, v, l1);
        } else {
            if constexpr (IN_LDS)
                dn_park_lds(v, l1);
            else
                stk[B] = v;
        }
    }
}

// What one task needs besides its rows.
struct DnTask {
    int nct, total;                  // column tiles, ring stages
    int64_t n0;                      // first output column
    __amdgpu_buffer_rsrc_t rb;       // the Wd rows of its column tiles
    uint32_t eoff[2];                // output byte offsets of this lane's two rows
};

// Per-call constants of the kernel.
struct DnCtx {
    __amdgpu_buffer_rsrc_t ra, re;   // h rows, e
    uint32_t voff[4];                // ring load offsets of this lane
    uint32_t lds_base, rowb, ch0, ch1, l1;
    char *lds;
    int64_t K;
};

// One k-step: 16 MFMAs on the fragments f and row k-step KSI; after MFMA m
// the fragment read m of fn (m < 8, when RD) and ring load m - 8 of stage
// dg (8 <= m < 12, when dm).
template <int KS, int KSI, bool FRESH, bool RD>
__device__ __forceinline__ void dn_kstep(DnAcc &acc, const DnRows<KS> &rows, const DnFrags &f,
                                         DnFrags &fn, uint32_t fa, bool dm, int dg,
                                         const DnTask &t, const DnCtx &x)
{
    static_for<16>([&](auto Mc) {
        constexpr int m = decltype(Mc)::value;
        constexpr int i = m / 8, j = m % 8;
        mfma_dn<FRESH>(acc.v[i][j], f.b[j], rows.v[i][KSI]);
        if constexpr (RD && m < 8)
            dn_frag<m>(fn, fa);
        if constexpr (m >= 8 && m < 12) {
            if (dm)
                dn_dma(t.rb, x.voff, x.lds, dg, KS / 2, x.K, m - 8);
        }
    });
}

// Stages of column tile c (ring stages g0 .. g0 + KS/2 - 1 of the task);
// on entry f0 holds the first k-step's fragments.  Loads of stage t are
// issued in the second k-step of stage t - 4 (the first four in the
// prologue), so at the barrier after the first k-step of stage g only the
// loads of stages g + 2 and g + 3 were issued after those of stage g + 1.
template <int KS, int LOG, int S>
__device__ __forceinline__ void dn_stages(DnAcc &acc, DnAcc (&stk)[LOG > 0 ? LOG : 1],
                                          const DnRows<KS> &rows, DnFrags &f0, DnFrags &f1,
                                          int g0, const DnTask &t, const DnCtx &x)
{
    constexpr int SPT = KS / 2;
    constexpr int LK = KS >> LOG;  // k-steps per leaf
    if constexpr (S < SPT) {
        const int g = g0 + S;
        const uint32_t bs = x.lds_base + (uint32_t)(g % kDnBuf) * kDnStage + x.rowb;
        dn_kstep<KS, 2 * S, (2 * S) % LK == 0, true>(acc, rows, f0, f1, bs + x.ch1, false, 0, t, x);
        dn_frags_wait(f1);
        dn_vm_barrier((g + 2 < t.total ? 4 : 0) + (g + 3 < t.total ? 4 : 0));
        const uint32_t bn = x.lds_base + (uint32_t)((g + 1) % kDnBuf) * kDnStage + x.rowb;
        dn_kstep<KS, 2 * S + 1, false, true>(acc, rows, f1, f0, bn + x.ch0, g + 4 < t.total, g + 4,
                                             t, x);
        dn_frags_wait(f0);
        if constexpr ((2 * S + 2) % LK == 0) {
            constexpr int J = (2 * S + 2) / LK - 1;  // the leaf just finished
            dn_drain(acc);
            dn_tree_push<LOG, J, 0>(stk, acc, x.l1);
        }
        dn_stages<KS, LOG, S + 1>(acc, stk, rows, f0, f1, g0, t, x);
    }
}

__device__ __forceinline__ DnTask dn_task(const MoeGemmArgs &a, const MoeTask &mt,
                                          int32_t (&ent)[2], int spt)
{
    DnTask t;
    const int rem = static_cast<int>((a.N - mt.n0 + 127) / 128);
    t.nct = rem < kDnCT ? rem : kDnCT;
    t.total = t.nct * spt;
    t.n0 = mt.n0;
    const int64_t boff = static_cast<int64_t>(mt.e) * a.N * a.K + mt.n0 * a.K;
    t.rb = tile_rsrc(a.B0 + boff, (int64_t)t.nct * 128, a.K);
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t ebytes = a.a_rows_total * a.N * 4;
    if (ebytes > 0xffffffffLL)
        ebytes = 0xffffffffLL;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = wave * 32 + i * 16 + (lane & 15);
        ent[i] = r < mt.nvalid ? a.rows[static_cast<int64_t>(mt.e) * a.T + mt.m0 + r] : -1;
        t.eoff[i] = ent[i] >= 0
                        ? (uint32_t)((int64_t)ent[i] * a.N * 4) + (uint32_t)(16 * (lane >> 4))
                        : (uint32_t)ebytes;
    }
    return t;
}

__device__ __forceinline__ void dn_row_bases(const MoeGemmArgs &a, const int32_t (&ent)[2],
                                             uint32_t (&base)[2])
{
    int64_t abytes = a.a_rows_total * a.K * 2;
    if (abytes > 0xffffffffLL)
        abytes = 0xffffffffLL;
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < 2; ++i)
        base[i] = ent[i] >= 0 ? (uint32_t)((int64_t)ent[i] * a.K * 2) + (uint32_t)((lane >> 4) * 16)
                              : (uint32_t)abytes;
}

// One task on the rows in `rows` (loads in flight; their first use waits).
template <int KS, int LOG>
__device__ __forceinline__ void dn_run(const DnTask &t, const DnCtx &x, const DnRows<KS> &rows)
{
    constexpr int SPT = KS / 2;
    for (int g = 0; g < 4; ++g)
        if (g < t.total)
            for (int q = 0; q < 4; ++q)
                dn_dma(t.rb, x.voff, x.lds, g, SPT, x.K, q);
    // stage 0 landed (the task's rows too: a use of them waits by itself)
    dn_vm_barrier((t.total > 1 ? 4 : 0) + (t.total > 2 ? 4 : 0) + (t.total > 3 ? 4 : 0));
    DnFrags f0, f1;
    dn_frag<0>(f0, x.lds_base + x.rowb + x.ch0);
    dn_frag<1>(f0, x.lds_base + x.rowb + x.ch0);
    dn_frag<2>(f0, x.lds_base + x.rowb + x.ch0);
    dn_frag<3>(f0, x.lds_base + x.rowb + x.ch0);
    dn_frag<4>(f0, x.lds_base + x.rowb + x.ch0);
    dn_frag<5>(f0, x.lds_base + x.rowb + x.ch0);
    dn_frag<6>(f0, x.lds_base + x.rowb + x.ch0);
    dn_frag<7>(f0, x.lds_base + x.rowb + x.ch0);
    dn_frags_wait(f0);
    for (int c = 0; c < t.nct; ++c) {
        DnAcc stk[LOG > 0 ? LOG : 1];
        DnAcc acc;
        dn_stages<KS, LOG, 0>(acc, stk, rows, f0, f1, c * SPT, t, x);
        const uint32_t soff = (uint32_t)((t.n0 + 128 * c) * 4);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(reinterpret_cast<const u32x4 &>(acc.v[i][j]),
                                                       x.re, t.eoff[i] + j * 64, soff, 0);
    }
    // every ring load has landed and every wave is done with the ring
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

// Persistent over the down tasks (the XCD-aware split of moe_expert_kernel),
// one workgroup of four waves per CU.
template <int KS, int LOG>
__global__ __launch_bounds__(256, 1) void moe_down_reg_kernel(MoeGemmArgs a,
                                                              const int32_t *__restrict__ tiles,
                                                              const int32_t *__restrict__ counts,
                                                              const int32_t *__restrict__ ntiles)
{
    static_assert((KS >> LOG) >= 2, "a leaf spans at least one ring stage");
    constexpr int SPT = KS / 2;
    constexpr int TN = 128 * kDnCT;
    __shared__ __attribute__((aligned(16))) char lds[kDnBuf * kDnStage + (LOG == 2 ? 4 * 16384 : 0)];
    const int ntn = static_cast<int>((a.N + TN - 1) / TN);
    const int total_tasks = __builtin_amdgcn_readfirstlane(*ntiles) * ntn;
    const int xcd = blockIdx.x % kXcds;
    const int slots = gridDim.x / kXcds;
    const int per = (total_tasks + kXcds - 1) / kXcds;
    const int end = (xcd + 1) * per < total_tasks ? (xcd + 1) * per : total_tasks;
    int w = xcd * per + static_cast<int>(blockIdx.x) / kXcds;
    if (w >= end)
        return;

    DnCtx x;
    x.K = a.K;
    x.lds = lds;
    x.lds_base = lds_addr(lds);
    {
        int64_t abytes = a.a_rows_total * a.K * 2;
        if (abytes > 0xffffffffLL)
            abytes = 0xffffffffLL;
        int64_t ebytes = a.a_rows_total * a.N * 4;
        if (ebytes > 0xffffffffLL)
            ebytes = 0xffffffffLL;
        x.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.A), (short)0,
                                                 (int)(uint32_t)abytes, 0x00020000);
        x.re = __builtin_amdgcn_make_buffer_rsrc(a.out, (short)0, (int)(uint32_t)ebytes, 0x00020000);
        const int lane = lane_id();
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const uint32_t c = (lane & 7) ^ (lane >> 3);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            x.voff[q] = (uint32_t)((int64_t)(32 * wave + 8 * q + (lane >> 3)) * a.K * 2) + c * 16;
        x.ch0 = (uint32_t)(((lane >> 4) ^ (lane & 7)) << 4);
        x.ch1 = x.ch0 ^ 64u;
        x.rowb = (uint32_t)(lane & 15) * kRowBytes;
        x.l1 = x.lds_base + kDnBuf * kDnStage + wave * 16384 + lane * 16;
    }

    DnRows<KS> rows;
    int32_t ent[2];
    uint32_t base[2];
    for (; w < end; w += slots) {
        const DnTask t = dn_task(a, moe_task(tiles, counts, w, ntn, TN), ent, SPT);
        dn_row_bases(a, ent, base);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                dn_row_load<KS>(rows, x.ra, base, i, ks);
        dn_run<KS, LOG>(t, x, rows);
    }
}

// --------------------------------------------------------------- combine

// y[t][n] = g_0 e_0 + g_1 e_1 + ... in routing order, left to right, each
// product rounded before its add.  Four consecutive n per thread.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float *gate, const float *eout,
                                                          float *y, int64_t T, int64_t H,
                                                          int top_k)
{
    const int64_t quads = T * (H / 4);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; q < quads;
         q += stride) {
        const int64_t t = q / (H / 4);
        const int64_t n = (q % (H / 4)) * 4;
        const float *g = gate + t * top_k;
        const float *e = eout + (t * top_k) * H + n;
        f32x4 acc = *reinterpret_cast<const f32x4 *>(e) * g[0];
        for (int k = 1; k < top_k; ++k) {
            const f32x4 prod = *reinterpret_cast<const f32x4 *>(e + k * H) * g[k];
            acc = acc + prod;
        }
        *reinterpret_cast<f32x4 *>(y + t * H + n) = acc;
    }
}

// ---------------------------------------------------------------- launch

template <int LOG, bool GU>
static void launch_expert(const MoeGemmArgs &a, hipStream_t stream)
{
    // eight waves with a three-stage ring (96 KiB) leave room for the
    // epilogue's own 32 KiB staging buffer
    using C = typename std::conditional<(LOG <= 1), CfgDual, TileCfg<4, 3>>::type;
    // resident workgroups, a multiple of 8
    const unsigned grid = static_cast<unsigned>(device_cus() / kXcds * kXcds * (LOG <= 1 ? 2 : 1));
    static_assert(kXcds == 8, "the task split assumes a grid that is a multiple of 8");
    hipLaunchKernelGGL((moe_expert_kernel<C, LOG, GU>), dim3(grid), dim3(C::kThreads), 0, stream,
                       a, a.tiles, a.counts, a.ntiles);
}

// Gate/up with at most four leaves over at least 16 stages takes the
// 128 x 256 tile; same bits as the 128 x 128 expert kernel.
template <int LOG>
static void launch_gu_wide(const MoeGemmArgs &a, hipStream_t stream)
{
    const unsigned grid = static_cast<unsigned>(device_cus() / kXcds * kXcds);
    hipLaunchKernelGGL((moe_gu_wide_kernel<LOG>), dim3(grid), dim3(256), 0, stream, a, a.tiles,
                       a.counts, a.ntiles);
}

template <bool GU>
static hipError_t dispatch_expert(const MoeGemmArgs &a, int leaves, hipStream_t stream)
{
    if (GU && leaves <= 4 && a.stages_per_leaf * leaves >= 16) {
        switch (leaves) {
        case 1: launch_gu_wide<0>(a, stream); break;
        case 2: launch_gu_wide<1>(a, stream); break;
        case 4: launch_gu_wide<2>(a, stream); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (leaves) {
    case 1: launch_expert<0, GU>(a, stream); break;
    case 2: launch_expert<1, GU>(a, stream); break;
    case 4: launch_expert<2, GU>(a, stream); break;
    case 8: launch_expert<3, GU>(a, stream); break;
    case 16: launch_expert<4, GU>(a, stream); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int KS, int LOG>
static void launch_down_reg(const MoeGemmArgs &a, hipStream_t stream)
{
    const unsigned grid = static_cast<unsigned>(device_cus() / kXcds * kXcds);
    hipLaunchKernelGGL((moe_down_reg_kernel<KS, LOG>), dim3(grid), dim3(256), 0, stream, a, a.tiles,
                       a.counts, a.ntiles);
}

// The down projection keeps a task's rows in registers when they fit
// (K = 128, 256 or 512), whole column tiles of 128 cover the output (H a
// multiple of 128) and a leaf spans at least one ring stage; otherwise the
// tile kernel.  Same bits either way.
static hipError_t dispatch_down(const MoeGemmArgs &a, int leaves, hipStream_t stream)
{
    const int KS = static_cast<int>(a.K / 32);
    // the register kernel addresses e (rows x N FP32) with 32-bit offsets; past
    // 4 GiB the expert kernel, which uses 64-bit pointers, takes the call
    const bool fits = (a.K == 128 || a.K == 256 || a.K == 512) && a.N % 128 == 0 &&
                      (leaves == 1 || leaves == 2 || leaves == 4) && KS / leaves >= 2 &&
                      a.a_rows_total * a.N * 4 <= 0xffffffffLL;
    if (!fits)
        return dispatch_expert<false>(a, leaves, stream);
    switch (KS * 8 + leaves) {
    case 4 * 8 + 1: launch_down_reg<4, 0>(a, stream); break;
    case 4 * 8 + 2: launch_down_reg<4, 1>(a, stream); break;
    case 8 * 8 + 1: launch_down_reg<8, 0>(a, stream); break;
    case 8 * 8 + 2: launch_down_reg<8, 1>(a, stream); break;
    case 8 * 8 + 4: launch_down_reg<8, 2>(a, stream); break;
    case 16 * 8 + 1: launch_down_reg<16, 0>(a, stream); break;
    case 16 * 8 + 2: launch_down_reg<16, 1>(a, stream); break;
    case 16 * 8 + 4: launch_down_reg<16, 2>(a, stream); break;
    default: return dispatch_expert<false>(a, leaves, stream);
    }
    return hipGetLastError();
}

hipError_t launch_moe(const uint16_t *X, const float *logits, const uint16_t *Wg,
                      const uint16_t *Wu, const uint16_t *Wd, float *Y, int64_t T, int64_t H,
                      int64_t E, int64_t I, int top_k, int gu_leaves, int gu_leaf_size,
                      int dn_leaves, int dn_leaf_size, const MoeBuffers &b, hipStream_t stream)
{
    const int Q = E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16;
    const dim3 rgrid(static_cast<unsigned>((T + 3) / 4));
    switch (Q) {
    case 1: hipLaunchKernelGGL(moe_route_kernel<1>, rgrid, dim3(256), 0, stream, logits, b.idx, b.gate, T, (int)E, top_k); break;
    case 2: hipLaunchKernelGGL(moe_route_kernel<2>, rgrid, dim3(256), 0, stream, logits, b.idx, b.gate, T, (int)E, top_k); break;
    case 4: hipLaunchKernelGGL(moe_route_kernel<4>, rgrid, dim3(256), 0, stream, logits, b.idx, b.gate, T, (int)E, top_k); break;
    case 8: hipLaunchKernelGGL(moe_route_kernel<8>, rgrid, dim3(256), 0, stream, logits, b.idx, b.gate, T, (int)E, top_k); break;
    default: hipLaunchKernelGGL(moe_route_kernel<16>, rgrid, dim3(256), 0, stream, logits, b.idx, b.gate, T, (int)E, top_k); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    if (b.nblk > 0) {
        hipLaunchKernelGGL(moe_bucket_count_kernel, dim3(static_cast<unsigned>(b.nblk)), dim3(1024),
                           0, stream, b.idx, b.blk_counts, T, (int)E, top_k);
        hipLaunchKernelGGL(moe_bucket_scatter_kernel, dim3(static_cast<unsigned>(b.nblk)),
                           dim3(1024), 0, stream, b.idx, b.blk_counts, b.rows, b.counts, T, (int)E,
                           top_k);
    } else {
        hipLaunchKernelGGL(moe_bucket_kernel, dim3(static_cast<unsigned>(E)), dim3(256), 0, stream,
                           b.idx, b.rows, b.counts, T * top_k, T);
    }
    hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(1024), 0, stream, b.counts, b.tiles,
                       b.ntiles, (int)E);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;

    MoeGemmArgs a;
    a.rows = b.rows;
    a.counts = b.counts;
    a.tiles = b.tiles;
    a.ntiles = b.ntiles;
    a.T = T;
    // gate/up: A = X rows (entry / top_k), B = Wg, Wu [E][I][H], out = h [T*k][I]
    a.A = X;
    a.a_rows_total = T;
    a.row_div = top_k;
    a.B0 = Wg;
    a.B1 = Wu;
    a.out = b.h;
    a.N = I;
    a.K = H;
    a.stages_per_leaf = gu_leaf_size / BK;
    if ((err = dispatch_expert<true>(a, gu_leaves, stream)) != hipSuccess)
        return err;
    // down: A = h rows (entry), B = Wd [E][H][I], out = e [T*k][H]
    a.A = b.h;
    a.a_rows_total = T * top_k;
    a.row_div = 1;
    a.B0 = Wd;
    a.B1 = nullptr;
    a.out = b.e;
    a.N = H;
    a.K = I;
    a.stages_per_leaf = dn_leaf_size / BK;
    if ((err = dispatch_down(a, dn_leaves, stream)) != hipSuccess)
        return err;
    const int64_t quads = T * (H / 4);
    int64_t blocks = (quads + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    if (blocks > 0)
        hipLaunchKernelGGL(moe_combine_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                           stream, b.gate, b.e, Y, T, H, top_k);
    return hipGetLastError();
}

// h[i] = bf16(silu(G[i]) U[i]) and, when act is given, act[i] = the FP32
// value before the rounding: the expert FFN's activation on its own, with
// the device function of the gate/up epilogue.
__global__ __launch_bounds__(256) void swiglu_kernel(const float *G, const float *U, float *act,
                                                     uint16_t *h, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += stride) {
        const float v = swiglu_act(G[i], U[i]);
        if (act)
            act[i] = v;
        h[i] = f32_to_bf16_rne(v);
    }
}

hipError_t launch_swiglu(const float *G, const float *U, float *act, uint16_t *h, int64_t n,
                         hipStream_t stream)
{
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    if (blocks > 0)
        hipLaunchKernelGGL(swiglu_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                           stream, G, U, act, h, n);
    return hipGetLastError();
}

}  // namespace iso
