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
#include "kernels.h"

namespace iso {

// ------------------------------------------------------------------ route

// Balanced tree over the 64 lanes of a wave in lane order (pairs (l, l^1),
// then (l, l^2), ...); every lane ends with the root.
__device__ __forceinline__ float wave_tree_sum(float v)
{
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1)
        v = v + shfl_xor(v, mask);
    return v;
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
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1)
        mx = fmaxf(mx, shfl_xor(mx, mask));

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
#pragma unroll
        for (int mask = 1; mask < 64; mask <<= 1) {
            const float ov = shfl_xor(bv, mask);
            const int oe = __shfl_xor(be, mask, 64);
            if (ov > bv || (ov == bv && oe < be)) {
                bv = ov;
                be = oe;
            }
        }
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
// idx[i] == e, in increasing i, into rows[e][0 .. count).  Each pass covers
// 2048 entries: thread j owns entries [8j, 8j + 8) of the pass; an exclusive
// scan of the per-thread match counts gives every match its ordered slot.
__global__ __launch_bounds__(256) void moe_bucket_kernel(const int32_t *idx, int32_t *rows,
                                                         int32_t *counts, int64_t n_entries,
                                                         int64_t T)
{
    __shared__ int scan[256];
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    int32_t *dst = rows + static_cast<int64_t>(e) * T;
    int count = 0;
    for (int64_t base = 0; base < n_entries; base += 2048) {
        const int64_t i0 = base + static_cast<int64_t>(tid) * 8;
        unsigned mask = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (i0 + j < n_entries && idx[i0 + j] == e)
                mask |= 1u << j;
        const int mine = __popc(mask);
        scan[tid] = mine;
        __syncthreads();
        // inclusive Hillis-Steele scan over the 256 counts
        for (int d = 1; d < 256; d <<= 1) {
            const int add = tid >= d ? scan[tid - d] : 0;
            __syncthreads();
            scan[tid] += add;
            __syncthreads();
        }
        int pos = count + scan[tid] - mine;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (mask & (1u << j))
                dst[pos++] = static_cast<int32_t>(i0 + j);
        count += scan[255];
        __syncthreads();
    }
    if (tid == 0)
        counts[e] = count;
}

// ------------------------------------------------------------------ plan

// Work list of (expert, first row) tiles in expert order: thread e (E <=
// 1024 threads) scans the per-expert tile counts and writes its own tiles.
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
    int n = scan[e] - mine;
    for (int m0 = 0; m0 < c; m0 += BM, ++n) {
        tiles[2 * n] = e;
        tiles[2 * n + 1] = m0;
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

// Pipe over gathered A rows: DMA row r of the tile reads source row
// rows_e[m0 + r] / row_div of the whole A matrix, or zero when r >= nvalid
// (its offset lies past the buffer's range).
template <class C>
__device__ __forceinline__ Pipe make_pipe_gather(const MoeGemmArgs &a, const int32_t *rows_e,
                                                 int m0, int nvalid, const uint16_t *B_tile,
                                                 int64_t rowsB)
{
    Pipe p = make_pipe<C>(a.A, 0, B_tile, rowsB, a.K, 0);
    p.ra = tile_rsrc(a.A, a.a_rows_total, a.K);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t c = (lane & 7) ^ (lane >> 3);
    const uint32_t oob = (uint32_t)(a.a_rows_total * a.K * 2);
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) {
        const int r = C::kDma * 8 * w + 8 * i + (lane >> 3);
        if (r < nvalid) {
            const int64_t src = rows_e[m0 + r] / a.row_div;
            p.voffa[i] = (uint32_t)(src * a.K * 2) + c * 16;
        } else {
            p.voffa[i] = oob;
        }
    }
    return p;
}

// Gate/up tiles hold 64 intermediate columns: B rows 0..63 of the tile are
// Wg rows n0..n0+63 (loaded by the first half of the waves) and B rows
// 64..127 are the same Wu rows (second half), so one contraction yields G in
// tile columns 0..63 and U in columns 64..127 of every row.
constexpr int kGuCols = BN / 2;

template <class C, int LOG, bool GATE_UP>
__global__ __launch_bounds__(C::kThreads, 2) void moe_expert_kernel(MoeGemmArgs a)
{
    __shared__ __attribute__((aligned(16))) char lds[C::kLdsBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / C::WC, wc = wave % C::WC;
    constexpr int TN = GATE_UP ? kGuCols : BN;  // output columns per tile
    const int ntn = static_cast<int>((a.N + TN - 1) / TN);
    const int total = __builtin_amdgcn_readfirstlane(*a.ntiles) * ntn;
    // XCD-aware work split: the workgroups on XCD x (blockIdx % 8 == x) take
    // the contiguous task range [x per, (x+1) per), so the tasks running
    // together on one L2 share an expert's weights and a tile's rows.  The
    // grid is a multiple of 8, so every task is taken exactly once.
    const int xcd = blockIdx.x % kXcds;
    const int slots = gridDim.x / kXcds;
    const int per = (total + kXcds - 1) / kXcds;
    const int end = (xcd + 1) * per < total ? (xcd + 1) * per : total;
    for (int w = xcd * per + static_cast<int>(blockIdx.x) / kXcds; w < end; w += slots) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // previous tile's stores drained
        const int tile = w / ntn;
        const int64_t n0 = static_cast<int64_t>(w % ntn) * TN;
        const int e = __builtin_amdgcn_readfirstlane(a.tiles[2 * tile]);
        const int m0 = __builtin_amdgcn_readfirstlane(a.tiles[2 * tile + 1]);
        const int cnt = __builtin_amdgcn_readfirstlane(a.counts[e]);
        const int nvalid = cnt - m0 < BM ? cnt - m0 : BM;
        const int32_t *rows_e = a.rows + static_cast<int64_t>(e) * a.T;
        const int64_t boff = static_cast<int64_t>(e) * a.N * a.K + n0 * a.K;

        Pipe p = make_pipe_gather<C>(a, rows_e, m0, nvalid, a.B0 + boff, a.N - n0);
        if constexpr (GATE_UP) {
            const int wu = __builtin_amdgcn_readfirstlane(wave);
            const int64_t brows = a.N - n0 < kGuCols ? a.N - n0 : kGuCols;
            p.rb = tile_rsrc((wu < C::kWaves / 2 ? a.B0 : a.B1) + boff, brows, a.K);
            const uint32_t c = (lane & 7) ^ (lane >> 3);
#pragma unroll
            for (int i = 0; i < C::kDma; ++i) {
                const uint32_t r = (C::kDma * 8 * wu + 8 * i + (lane >> 3)) & (kGuCols - 1);
                p.voffb[i] = (uint32_t)((int64_t)r * a.K * 2) + c * 16;
            }
        }
        Acc<C> r0;
        leaf_tree_mainloop<C, LOG>(p, a.stages_per_leaf, lds, r0);

        if constexpr (GATE_UP) {
            // h = bf16(silu(G) * U), G in tile columns 0..63, U in 64..127.
            const float *stage = stage_tile<C>(r0, lds);
            const float kLog2e = 1.44269504088896340736f;
            uint16_t *o = static_cast<uint16_t *>(a.out) + n0;
            const bool al = (reinterpret_cast<uintptr_t>(o) % 16 == 0) && (a.N % 8 == 0);
            const int cmax = a.N - n0 < kGuCols ? static_cast<int>(a.N - n0) : kGuCols;
            for (int u = threadIdx.x; u < BM * (kGuCols / 8); u += C::kThreads) {
                const int row = u >> 3, q = u & 7;
                if (row >= nvalid)
                    break;
                const f32x4 g0 = staged_chunk(stage, row, 2 * q);
                const f32x4 g1 = staged_chunk(stage, row, 2 * q + 1);
                const f32x4 u0 = staged_chunk(stage, row, kGuCols / 4 + 2 * q);
                const f32x4 u1 = staged_chunk(stage, row, kGuCols / 4 + 2 * q + 1);
                const float gs[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
                const float us[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float ex = __builtin_amdgcn_exp2f(-gs[e] * kLog2e);
                    const float sg = gs[e] / (1.0f + ex);
                    v[e] = sg * us[e];
                }
                const int64_t dst = rows_e[m0 + row];
                store8_bf16(o + dst * a.N + 8 * q, v, al && 8 * q + 8 <= cmax, cmax - 8 * q);
            }
        } else {
            store_tile<C>(r0, lds, static_cast<float *>(a.out) + n0, a.N, nvalid, a.N - n0, false,
                          rows_e + m0);
        }
        __syncthreads();  // the next tile's loads overwrite the LDS
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
    using C = typename std::conditional<(LOG <= 1), CfgDual, CfgWide>::type;
    // resident workgroups, a multiple of 8
    const unsigned grid = static_cast<unsigned>(device_cus() / kXcds * kXcds * (LOG <= 1 ? 2 : 1));
    static_assert(kXcds == 8, "the task split assumes a grid that is a multiple of 8");
    hipLaunchKernelGGL((moe_expert_kernel<C, LOG, GU>), dim3(grid), dim3(C::kThreads), 0, stream,
                       a);
}

template <bool GU>
static hipError_t dispatch_expert(const MoeGemmArgs &a, int leaves, hipStream_t stream)
{
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
    hipLaunchKernelGGL(moe_bucket_kernel, dim3(static_cast<unsigned>(E)), dim3(256), 0, stream,
                       b.idx, b.rows, b.counts, T * top_k, T);
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
    if ((err = dispatch_expert<false>(a, dn_leaves, stream)) != hipSuccess)
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

}  // namespace iso
