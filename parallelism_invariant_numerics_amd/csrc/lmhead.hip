// lmhead.hip -- fused LM-head log-softmax statistics and sampled-token
// logprob for gfx950.
//
// The rollout engine records the sampled token's logprob and the trainer
// recomputes it (katelyatop-blog post on vLLM/SkyRL IsoExec, section 1 and
// section 4); both must see the same bits, so the softmax reduction is a
// fixed tree too ("IsoExec: Eliminating Trainer-Inference Mismatch in SkyRL",
// section "Achieving Parallelism Invariance": partials are combined by a
// fixed binary tree regardless of layout).
//
// Tree over the vocabulary:
//   chunk = 128 consecutive token ids = one workgroup tile's columns;
//   chunk max: exact (order-free);
//   chunk sum of exp(z - chunk max): balanced binary tree over the 128 ids in
//     index order -- lanes (l, l^1), (l, l^2), (l, l^4), (l, l^8) hold
//     neighbouring columns of a 16-wide MFMA block, then the four blocks of a
//     wave pair up in registers, then the two waves through LDS;
//   chunk merge: balanced binary tree over chunk index with the (m, s) merge
//     of device_common.hpp, padded with (-inf, 0).
// The logits never leave registers on the fused path (one partition).  With
// several partitions the partition roots of the logits go through the
// workspace and the same epilogue function runs on their folded values.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "gemm_core.hpp"
#include "kernels.h"

namespace iso {

constexpr int kChunk = BN;  // 128 token ids per chunk = one tile's columns

struct LmArgs {
    const uint16_t *H;
    const uint16_t *Wvt;
    const int32_t *tok;
    float *stats;   // [M][stats_stride][2]
    float *target;  // [M]
    const float *roots;  // [parts][M][V] (several partitions only)
    int64_t M, V, K, nchunk;  // V, nchunk: this call's vocabulary (a shard or all of it)
    int64_t v0;               // first token id of this call's vocabulary
    int64_t chunk0;           // its first chunk in the whole vocabulary
    int64_t stats_stride;     // chunks of the whole vocabulary (stats row stride)
    int stages_per_leaf;
};

// Chunk statistics of one 128 x 128 logit tile held in MFMA layout.  The
// chunk's columns are spread over the C::WC waves of a tile row; every launch
// shape reduces them with the same balanced tree in column order (16-column
// blocks by lane butterfly, then blocks inside a wave, then waves), so the
// bits do not depend on the shape.  `red` is LDS scratch of at least
// 2 * C::WC * 128 floats, free for use on entry.
template <class C>
__device__ __forceinline__ float tree_blocks(const float (&b)[C::JB])
{
    if constexpr (C::JB == 4)
        return (b[0] + b[1]) + (b[2] + b[3]);
    else
        return b[0] + b[1];
}

template <class C>
__device__ __forceinline__ float tree_waves(const float *red, int rt)
{
    if constexpr (C::WC == 4)
        return (red[rt] + red[128 + rt]) + (red[256 + rt] + red[384 + rt]);
    else
        return red[rt] + red[128 + rt];
}

// `tok_s` holds the tile rows' sampled token ids in LDS (written before the
// first barrier below, by any thread).
template <class C>
__device__ __forceinline__ void chunk_stats_epilogue(const Acc<C> &z, int64_t m0, int64_t n0,
                                                     const LmArgs &a, float *red,
                                                     const int32_t *tok_s)
{
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / C::WC, wc = wave % C::WC;
    const int64_t chunk = n0 / kChunk;
    float *red_m = red;
    float *red_s = red + C::WC * 128;

    bool colv[C::JB];
#pragma unroll
    for (int j = 0; j < C::JB; ++j)
        colv[j] = n0 + tile_col<C>(lane, wc, j) < a.V;

    // per-wave maxima per row, then the chunk maximum (exact, order-free)
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float m = -INFINITY;
#pragma unroll
            for (int j = 0; j < C::JB; ++j)
                if (colv[j])
                    m = fmaxf(m, z.v[i][j][r]);
            m = row16_max(m);
            if ((lane & 15) == 0)
                red_m[wc * 128 + tile_row<C>(lane, wr, i, r)] = m;
        }
    lds_barrier();

    // exp-sums: 16-column blocks by lane butterfly, then blocks, then waves;
    // the chunk maximum of each row is read back where it is needed
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rt = tile_row<C>(lane, wr, i, r);
            float cm = red_m[rt];
#pragma unroll
            for (int q = 1; q < C::WC; ++q)
                cm = fmaxf(cm, red_m[q * 128 + rt]);
            float blk[C::JB];
#pragma unroll
            for (int j = 0; j < C::JB; ++j) {
                const float e = colv[j] ? exp_neg(z.v[i][j][r] - cm) : 0.0f;
                blk[j] = row16_sum(e);
            }
            const float part = tree_blocks<C>(blk);
            if ((lane & 15) == 0)
                red_s[wc * 128 + tile_row<C>(lane, wr, i, r)] = part;
        }
    lds_barrier();

    if (wc == 0 && (lane & 15) == 0) {
#pragma unroll
        for (int i = 0; i < C::IB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rt = tile_row<C>(lane, wr, i, r);
                const int64_t row = m0 + rt;
                if (row < a.M) {
                    float cm = red_m[rt];
#pragma unroll
                    for (int q = 1; q < C::WC; ++q)
                        cm = fmaxf(cm, red_m[q * 128 + rt]);
                    float *st = a.stats + (row * a.stats_stride + a.chunk0 + chunk) * 2;
                    st[0] = cm;
                    st[1] = tree_waves<C>(red_s, rt);
                }
            }
    }

    // the sampled token's logit: written by the one lane that holds it
    constexpr int WCOLS = BN / C::WC;
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rt = tile_row<C>(lane, wr, i, r);
            const int64_t row = m0 + rt;
            if (row >= a.M)
                continue;
            const int64_t t = tok_s[rt] - a.v0;  // token id within this call's vocabulary
            const int64_t rel = t - n0 - wc * WCOLS - (lane & 15);
            if (rel >= 0 && rel < WCOLS && (rel & 15) == 0 && t < a.V) {
                const int j = static_cast<int>(rel >> 4);
                // a select chain: an indexed read of z would put the tile in
                // private memory
                float zt = z.v[i][0][r];
#pragma unroll
                for (int jj = 1; jj < C::JB; ++jj)
                    zt = j == jj ? z.v[i][jj][r] : zt;
                a.target[row] = zt;
            }
        }
}

// Tile order of the LM-head: groups of kLmColGroup vocabulary tiles, tile
// columns fastest inside a group, then the next row tile.  Each XCD takes a
// contiguous stretch of this order, i.e. its own eighth of the vocabulary for
// every row, so the 622 MB vocabulary matrix streams through one L2 instead
// of all eight, and only the hidden rows (34 MB) are shared.  The 32 tiles
// that run together on an XCD are 4 vocabulary tiles x 8 row tiles.
constexpr int kLmColGroup = 4;

// Origin and operand pipe of tile t of that order.
template <class C>
__device__ __forceinline__ Pipe lm_tile(const LmArgs &a, int t, int tm, int tn, int64_t &m0,
                                        int64_t &n0)
{
    int mt, nt;
    grouped_tile(t, tn, tm, kLmColGroup, nt, mt);
    m0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(mt)) * BM;
    n0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(nt)) * BN;
    return make_pipe<C>(a.H + m0 * a.K, a.M - m0, a.Wvt + n0 * a.K, a.V - n0, a.K, 0);
}

// The sampled token ids of tile rows m0 .. m0+127 into dst (LDS), by direct
// global-to-LDS loads of the first two waves; rows at or past M read as 0
// (they are never used).  Tracked by the vector memory counter like the
// operand stages.
__device__ __forceinline__ void tok_dma(const LmArgs &a, int64_t m0, int32_t *dst)
{
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w < BM / 64) {
        const int64_t rows = a.M - m0 < BM ? a.M - m0 : BM;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t *>(a.tok + m0), (short)0, static_cast<int>(rows * 4), 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ISO_LDS void *)(dst + 64 * w), 4,
                                                 static_cast<uint32_t>(lane_id() * 4),
                                                 static_cast<uint32_t>(w * 256), 0, 0);
    }
}

// Persistent: the workgroups on XCD x take the contiguous range
// [x per, (x+1) per) of the LM-head tile order (so the tiles running together
// on one L2 share hidden rows and vocabulary rows, and each vocabulary tile is
// needed by one XCD only), stepping by the number of workgroups per XCD.  The next tile's first stages and token ids are
// requested before the current tile's softmax epilogue, which hides their
// latency.  Nothing but loads to LDS is in flight across the epilogue, and
// nothing is carried in vector registers from one tile to the next.
template <class C, int LOG>
__global__ __launch_bounds__(C::kThreads, 2) void lmhead_fused_kernel(LmArgs a)
{
    __shared__ __attribute__((aligned(16))) char lds[C::kLdsBytes];
    __shared__ float red[2 * C::WC * 128];
    __shared__ int32_t tok_s[2][BM];
    const int tm = static_cast<int>((a.M + BM - 1) / BM);
    const int tn = static_cast<int>(a.nchunk);
    const int total = tm * tn;
    const int xcd = blockIdx.x % kXcds;
    const int slots = gridDim.x / kXcds;
    const int per = (total + kXcds - 1) / kXcds;
    const int end = (xcd + 1) * per < total ? (xcd + 1) * per : total;
    int w = xcd * per + static_cast<int>(blockIdx.x) / kXcds;
    if (w >= end)
        return;
    const int nst = (1 << LOG) * a.stages_per_leaf;

    int64_t m0, n0;
    {
        const Pipe p0 = lm_tile<C>(a, w, tm, tn, m0, n0);
        tok_dma(a, m0, tok_s[0]);
        pipe_prologue<C>(p0, lds, nst);
    }
    for (int it = 0;; ++it) {
        Acc<C> z;
        {
            const Pipe pipe = lm_tile<C>(a, w, tm, tn, m0, n0);
            leaf_tree_mainloop<C, LOG, false>(pipe, a.stages_per_leaf, lds, z);
        }
        const int wn = w + slots;
        if (wn < end) {
            int64_t m0n, n0n;
            const Pipe pn = lm_tile<C>(a, wn, tm, tn, m0n, n0n);
            tok_dma(a, m0n, tok_s[(it + 1) & 1]);
            pipe_prologue<C>(pn, lds, nst);
        }
        chunk_stats_epilogue<C>(z, m0, n0, a, red, tok_s[it & 1]);
        if (wn >= end)
            break;
        w = wn;
    }
}

// ------------------------------------------------------ decode (M <= 16 rows)
//
// A decode step evaluates one to 16 rows against the whole vocabulary: the
// 622 MB vocabulary matrix is read once and the rows fill a single 16-row
// MFMA block.  The work is the same as the fused kernel's for those rows (the
// same v_mfma_f32_16x16x32_bf16 chain per leaf in ascending k, the same
// balanced tree over the leaves, the same chunk statistics), so the bits are
// those of the fused kernel; only the data movement differs.  One workgroup
// of 8 waves per CU walks the chunks (128 vocabulary ids each) in a
// grid-stride loop.  Wave w takes the 16 ids n0 + 16 w .. + 15 and all the
// leaves, folded by the register tree.  Weight fragments go from HBM straight
// to registers, one leaf (KS k-steps) ahead, so a CU keeps 8 x KS KiB of
// weights in flight (16 waves, each on half of the leaves, kept twice as
// much in flight and took 2-4 % longer); the rows (zero past M) sit in LDS
// for the whole launch.  The chunk statistics use the balanced tree over the
// eight 16-id blocks in id order, which is the fused kernel's tree.
constexpr int kDecRows = 16;
constexpr int kDecWaves = 8;
constexpr int64_t kDecMaxK = 4096;
constexpr int kDecPitchMax = static_cast<int>(kDecMaxK) * 2 + 16;  // LDS bytes per row

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v)
{
    return __builtin_bit_cast(bf16x8, v);
}

template <int LOG, int KS>
__global__ __launch_bounds__(kDecWaves * 64) void lmhead_decode_kernel(LmArgs a)
{
    static_assert(LOG >= 1, "an even number of leaves");
    constexpr int LH = 1 << LOG;  // leaves (even: leaf 0 of the next chunk lands in buffer 0)
    __shared__ __attribute__((aligned(16))) char arow[kDecRows * kDecPitchMax];
    __shared__ float red_m[8][kDecRows], red_s[8][kDecRows];

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int blk = wave;
    const int64_t K = a.K;
    const int pitch = static_cast<int>(K) * 2 + 16;  // 16 bytes of padding: rows shift banks

    // the rows into LDS (rows M .. 15 zero), 16 bytes per thread and step
    {
        const int per_row = static_cast<int>(K / 8);
        for (int q = threadIdx.x; q < kDecRows * per_row; q += kDecWaves * 64) {
            const int r = q / per_row, c = q % per_row;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (r < a.M)
                v = *reinterpret_cast<const u32x4 *>(a.H + static_cast<int64_t>(r) * K + 8 * c);
            *reinterpret_cast<u32x4 *>(arow + r * pitch + 16 * c) = v;
        }
    }
    __syncthreads();

    int64_t c = blockIdx.x;
    if (c >= a.nchunk)
        return;  // the whole workgroup
    // this lane's A fragment row (lane & 15) and k-group (lane >> 4); its B
    // row (lane & 15) of the wave's 16 ids and the same k-group
    const uint32_t a_lds = lds_addr(arow) + static_cast<uint32_t>((lane & 15) * pitch + (lane >> 4) * 16);
    const uint32_t voff = static_cast<uint32_t>((lane & 15) * K * 2 + (lane >> 4) * 16);

    auto brsrc = [&](int64_t ch) {
        const int64_t col0 = ch * kChunk + 16 * blk;
        int64_t rows = a.V - col0;
        rows = rows < 0 ? 0 : (rows > 16 ? 16 : rows);
        return tile_rsrc(a.Wvt + (rows > 0 ? col0 : 0) * K, rows, K);
    };
    auto load_leaf = [&](u32x4 (&dst)[KS], __amdgpu_buffer_rsrc_t r, int leaf) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            dst[kk] = __builtin_amdgcn_raw_buffer_load_b128(
                r, voff, static_cast<int>((leaf * KS + kk) * 64), 0);
    };

    u32x4 bb[2][KS];
    __amdgpu_buffer_rsrc_t rb = brsrc(c);
    load_leaf(bb[0], rb, 0);
    for (;;) {
        const int64_t cn = c + gridDim.x;
        const __amdgpu_buffer_rsrc_t rbn = brsrc(cn < a.nchunk ? cn : c);
        f32x4 stk[LOG];
        f32x4 acc;
        static_for<LH>([&](auto Jc) {
            constexpr int J = decltype(Jc)::value;
            constexpr int cur = J & 1;
            // the next leaf of this chunk, or leaf 0 of the next chunk (LH is
            // even, so that one lands in buffer 0)
            if constexpr (J + 1 < LH)
                load_leaf(bb[cur ^ 1], rb, J + 1);
            else if (cn < a.nchunk)
                load_leaf(bb[cur ^ 1], rbn, 0);
            acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                f32x4 av;
                lds_issue_b128(av, a_lds + static_cast<uint32_t>((J * KS + kk) * 64));
                lds_wait();
                lds_pin(av);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                              as_bf16x8(bb[cur][kk]), acc, 0, 0, 0);
            }
            // binary-counter tree over the leaves (lower leaves left)
            bool done = false;
#pragma unroll
            for (int b = 0; b < LOG; ++b) {
                if (!done) {
                    if ((J >> b) & 1) {
                        acc = stk[b] + acc;
                    } else {
                        stk[b] = acc;
                        done = true;
                    }
                }
            }
        });

        // epilogue: the chunk statistics (the barrier first: wave 0 has read
        // the previous chunk's block maxima and sums)
        lds_barrier();
        const int64_t n0 = c * kChunk;
        const int64_t col = n0 + 16 * blk + (lane & 15);
        const bool colv = col < a.V;
        const f32x4 z = acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float m = colv ? z[r] : -INFINITY;
            m = row16_max(m);
            if ((lane & 15) == 0)
                red_m[blk][4 * (lane >> 4) + r] = m;
        }
        lds_barrier();
        {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * (lane >> 4) + r;
                float cm = red_m[0][row];
#pragma unroll
                for (int q = 1; q < 8; ++q)
                    cm = fmaxf(cm, red_m[q][row]);
                const float e = colv ? exp_neg(z[r] - cm) : 0.0f;
                const float sblk = row16_sum(e);
                if ((lane & 15) == 0)
                    red_s[blk][row] = sblk;
                if (row < a.M) {
                    const int64_t t = static_cast<int64_t>(a.tok[row]) - a.v0;
                    if (t == col && t < a.V)
                        a.target[row] = z[r];
                }
            }
        }
        lds_barrier();
        if (wave == 0 && (lane & 15) == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * (lane >> 4) + r;
                if (row < a.M) {
                    float cm = red_m[0][row];
#pragma unroll
                    for (int q = 1; q < 8; ++q)
                        cm = fmaxf(cm, red_m[q][row]);
                    const float sum = ((red_s[0][row] + red_s[1][row]) + (red_s[2][row] + red_s[3][row])) +
                                      ((red_s[4][row] + red_s[5][row]) + (red_s[6][row] + red_s[7][row]));
                    float *st = a.stats + (row * a.stats_stride + a.chunk0 + c) * 2;
                    st[0] = cm;
                    st[1] = sum;
                }
            }
        }
        if (cn >= a.nchunk)
            break;
        c = cn;
        rb = rbn;
    }
}

template <int LOG, int KS>
static hipError_t launch_decode(const LmArgs &a, hipStream_t stream)
{
    int64_t g = device_cus();
    g = a.nchunk < g ? a.nchunk : g;
    hipLaunchKernelGGL((lmhead_decode_kernel<LOG, KS>), dim3(static_cast<unsigned>(g)),
                       dim3(kDecWaves * 64), 0, stream, a);
    return hipGetLastError();
}

// The decode kernel when it applies (one partition, M <= 16, four or eight
// leaves of 64, 128 or 256 columns, K <= 4096); hipErrorNotSupported
// otherwise (the fused kernel takes those).
static hipError_t try_decode(const LmArgs &a, int leaves, int leaf_size, hipStream_t stream)
{
    if (a.M < 1 || a.M > kDecRows || a.K > kDecMaxK)
        return hipErrorNotSupported;
    const int ks = leaf_size / 32;
    if (leaves == 4) {
        switch (ks) {
        case 2: return launch_decode<2, 2>(a, stream);
        case 4: return launch_decode<2, 4>(a, stream);
        case 8: return launch_decode<2, 8>(a, stream);
        default: return hipErrorNotSupported;
        }
    }
    if (leaves == 8) {
        switch (ks) {
        case 2: return launch_decode<3, 2>(a, stream);
        case 4: return launch_decode<3, 4>(a, stream);
        case 8: return launch_decode<3, 8>(a, stream);
        default: return hipErrorNotSupported;
        }
    }
    return hipErrorNotSupported;
}

// Several partitions: fold the partition roots of the logits with the top
// tree levels, in the MFMA layout, then the same epilogue.
template <int P>
__global__ __launch_bounds__(CfgDual::kThreads) void lmhead_roots_kernel(LmArgs a)
{
    using C = CfgDual;
    __shared__ float red[2 * C::WC * 128];
    __shared__ int32_t tok_s[BM];
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BN;
    if (threadIdx.x < BM)
        tok_s[threadIdx.x] = m0 + threadIdx.x < a.M ? a.tok[m0 + threadIdx.x] : -1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / C::WC, wc = wave % C::WC;
    const int64_t MV = a.M * a.V;
    Acc<C> z;
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
#pragma unroll
        for (int j = 0; j < C::JB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int64_t row = m0 + tile_row<C>(lane, wr, i, r);
                int64_t col = n0 + tile_col<C>(lane, wc, j);
                row = row < a.M ? row : a.M - 1;
                col = col < a.V ? col : a.V - 1;
                float rv[P];
#pragma unroll
                for (int q = 0; q < P; ++q)
                    rv[q] = a.roots[q * MV + row * a.V + col];
                z.v[i][j][r] = fold_roots<P>(rv);
            }
    chunk_stats_epilogue<C>(z, m0, n0, a, red, tok_s);
}

// Per row: balanced tree over the chunk statistics in chunk order, then
// logprob = (z_t - max) - log(sum).  One 256-thread workgroup per row;
// thread t folds chunks [t*PER, (t+1)*PER), then lanes and waves pair up.
template <int PER>
__global__ __launch_bounds__(256) void lmhead_finish_kernel(const float *stats,
                                                            const float *target,
                                                            const int32_t *tok, float *logprob,
                                                            int64_t M, int64_t V, int64_t nchunk)
{
    __shared__ float wm[4], ws[4];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    float m[PER], s[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int64_t c = static_cast<int64_t>(tid) * PER + q;
        if (c < nchunk) {
            m[q] = stats[(row * nchunk + c) * 2 + 0];
            s[q] = stats[(row * nchunk + c) * 2 + 1];
        } else {
            m[q] = -INFINITY;
            s[q] = 0.0f;
        }
    }
#pragma unroll
    for (int width = PER; width > 1; width >>= 1)
#pragma unroll
        for (int q = 0; q < width / 2; ++q) {
            float mm = m[2 * q], ss = s[2 * q];
            lse_merge(mm, ss, m[2 * q + 1], s[2 * q + 1]);
            m[q] = mm;
            s[q] = ss;
        }
    float mv = m[0], sv = s[0];
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) {
        const float m2 = shfl_xor(mv, mask);
        const float s2 = shfl_xor(sv, mask);
        lse_merge(mv, sv, m2, s2);
    }
    if ((tid & 63) == 0) {
        wm[tid >> 6] = mv;
        ws[tid >> 6] = sv;
    }
    lds_barrier();
    if (tid == 0) {
        float m01 = wm[0], s01 = ws[0];
        lse_merge(m01, s01, wm[1], ws[1]);
        float m23 = wm[2], s23 = ws[2];
        lse_merge(m23, s23, wm[3], ws[3]);
        lse_merge(m01, s01, m23, s23);
        const int64_t t = tok[row];
        float lp;
        if (t < 0 || t >= V)
            lp = __builtin_nanf("");
        else
            lp = (target[row] - m01) - log_f32(s01);
        logprob[row] = lp;
    }
}

template <int LOG>
static hipError_t launch_fused(const LmArgs &a, hipStream_t stream)
{
    using C = typename std::conditional<(LOG <= 1), CfgDual, CfgWide>::type;
    const int64_t tiles = ((a.M + BM - 1) / BM) * a.nchunk;
    const int64_t slots = static_cast<int64_t>(device_cus()) * (C::kWaves == 4 ? 2 : 1);
    int64_t g = tiles < slots ? tiles : slots;
    g = (g + kXcds - 1) / kXcds * kXcds;  // whole rounds over the XCDs
    dim3 grid(static_cast<unsigned>(g));
    hipLaunchKernelGGL((lmhead_fused_kernel<C, LOG>), grid, dim3(C::kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_lmhead_stats(const uint16_t *H, const uint16_t *Wvt, const int32_t *tok,
                               float *ws_stats, float *ws_target, float *ws_roots, int64_t M,
                               int64_t V, int64_t K, int leaves_per_part, int leaf_size,
                               int parts, int64_t v0, int64_t v_total, hipStream_t stream)
{
    LmArgs a;
    a.H = H;
    a.Wvt = Wvt;
    a.tok = tok;
    a.stats = ws_stats;
    a.target = ws_target;
    a.roots = ws_roots;
    a.M = M;
    a.V = V;
    a.K = K;
    a.nchunk = (V + kChunk - 1) / kChunk;
    a.v0 = v0;
    a.chunk0 = v0 / kChunk;
    a.stats_stride = (v_total + kChunk - 1) / kChunk;
    a.stages_per_leaf = leaf_size / BK;
    if (parts == 1) {
        const hipError_t d = try_decode(a, leaves_per_part, leaf_size, stream);
        if (d != hipErrorNotSupported)
            return d;
        switch (leaves_per_part) {
        case 1: return launch_fused<0>(a, stream);
        case 2: return launch_fused<1>(a, stream);
        case 4: return launch_fused<2>(a, stream);
        case 8: return launch_fused<3>(a, stream);
        case 16: return launch_fused<4>(a, stream);
        default: return hipErrorInvalidValue;
        }
    }
    hipError_t e = launch_gemm_partials(H, Wvt, ws_roots, 2, M, V, K, leaves_per_part, leaf_size,
                                        parts, stream);
    if (e != hipSuccess)
        return e;
    dim3 grid(static_cast<unsigned>((M + BM - 1) / BM), static_cast<unsigned>(a.nchunk));
    switch (parts) {
    case 2: hipLaunchKernelGGL(lmhead_roots_kernel<2>, grid, dim3(CfgDual::kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(lmhead_roots_kernel<4>, grid, dim3(CfgDual::kThreads), 0, stream, a); break;
    case 8: hipLaunchKernelGGL(lmhead_roots_kernel<8>, grid, dim3(CfgDual::kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The workspace of iso_lmhead_logprob_noalloc: chunk statistics and target
// logits of one call, for callers that cannot allocate.  Every GPU the
// library runs on holds its own copy until the process ends; calls that
// overlap on one GPU share it and race.  Nothing in it needs clearing: a
// call writes every chunk pair of its rows before the finish kernel reads
// them, and reads a target logit only for a token id it has written.
static __device__ __align__(256) char scratch[kLmNoallocBytes];

hipError_t lmhead_noalloc_scratch(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<void *> addr[kMaxDevices];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            // with `dev` current: each GPU's copy has its own address; the
            // name `scratch` itself is a host-side stand-in, never passed on
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            if (!p)
                return hipErrorInvalidSymbol;
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_lmhead_finish(const float *ws_stats, const float *ws_target,
                                const int32_t *tok, float *logprob, int64_t M, int64_t V,
                                hipStream_t stream)
{
    const int64_t nchunk = (V + kChunk - 1) / kChunk;
    int64_t pad = 256;
    while (pad < nchunk)
        pad <<= 1;
    const int64_t per = pad / 256;
    dim3 grid(static_cast<unsigned>(M));
    switch (per) {
    case 1: hipLaunchKernelGGL(lmhead_finish_kernel<1>, grid, dim3(256), 0, stream, ws_stats, ws_target, tok, logprob, M, V, nchunk); break;
    case 2: hipLaunchKernelGGL(lmhead_finish_kernel<2>, grid, dim3(256), 0, stream, ws_stats, ws_target, tok, logprob, M, V, nchunk); break;
    case 4: hipLaunchKernelGGL(lmhead_finish_kernel<4>, grid, dim3(256), 0, stream, ws_stats, ws_target, tok, logprob, M, V, nchunk); break;
    case 8: hipLaunchKernelGGL(lmhead_finish_kernel<8>, grid, dim3(256), 0, stream, ws_stats, ws_target, tok, logprob, M, V, nchunk); break;
    case 16: hipLaunchKernelGGL(lmhead_finish_kernel<16>, grid, dim3(256), 0, stream, ws_stats, ws_target, tok, logprob, M, V, nchunk); break;
    case 32: hipLaunchKernelGGL(lmhead_finish_kernel<32>, grid, dim3(256), 0, stream, ws_stats, ws_target, tok, logprob, M, V, nchunk); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace iso
