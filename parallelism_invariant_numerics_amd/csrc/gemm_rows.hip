// gemm_rows.hip -- the leaf/tree GEMM for calls of a few rows up to a few
// hundred (decode steps and small batches of a linear layer), for gfx950.
//
// Numerics: those of gemm_core.hpp ("IsoExec: Eliminating Trainer-Inference
// Mismatch in SkyRL", section "Achieving Parallelism Invariance", TP bullet:
// contiguous K leaves, FP32 accumulation, one fixed binary tree).  Each leaf
// sum is the same chain of v_mfma_f32_16x16x32_bf16 steps in ascending k,
// started from +0.0, and the leaves are combined by the same balanced tree,
// so an element has the bits the tile kernels give it in any batch.
//
// Why a kernel of its own: with few rows the work is the weight stream
// (N x K bf16), and a 128 x 128 output tile per workgroup leaves all but
// (M / 128) (N / 128) CUs idle.  Here a workgroup of eight waves takes 16
// output columns (two blocks of 16 for four leaves); wave w of a block takes
// the contiguous subtree of L / S leaves number w (S = 8, or 4 for four
// leaves) and loads all of its weight fragments into registers once.  The
// rows then pass through in groups of 16 (one MFMA row block), double-
// buffered: while a group multiplies, the next group's row fragments of the
// wave's K range load into the other register set.  The wave folds its
// leaves with the register tree, and the S subtree roots meet in LDS, where
// the top log2 S tree levels combine them in index order.  Every row group
// reuses the weights in registers, so the weights leave HBM once per call.
#include "gemm_core.hpp"
#include "kernels.h"

namespace iso {


// The per-wave state of one column block: its weight fragments (all of its
// subtree's K range) and where its rows and outputs are.
template <int NK>
struct RowsWave {
    u32x4 bf[NK];
    uint32_t voff;  // this lane's byte offset in a 16-row block of A / Wt
    int k0;         // first k-step of the wave's subtree
    int64_t col;    // this lane's output column
    int sub, cb, wave, lane;
};

// Issue the loads of the wave's row fragments of rows r0 .. r0+15 (rows past
// M read as zero).  No wait: the caller's first use of `af` waits.
template <int NK>
__device__ __forceinline__ void rows_load(u32x4 (&af)[NK], const RowsWave<NK> &w,
                                          const uint16_t *A, int64_t M, int64_t K, int64_t r0)
{
    const __amdgpu_buffer_rsrc_t ra = tile_rsrc(A + r0 * K, M - r0, K);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
        af[kk] = __builtin_amdgcn_raw_buffer_load_b128(ra, w.voff, (w.k0 + kk) * 64, 0);
}

// One 16-row group: the wave's leaves by MFMA chains and the register tree,
// the subtree roots through LDS, the top tree levels and the store.  Ends
// with every wave past the roots buffer, so the next group may reuse it;
// LDS-only barriers, so the next group's row loads stay in flight.
template <int S, int LWLOG, int KS, int NK>
__device__ __forceinline__ void rows_group(const u32x4 (&af)[NK], const RowsWave<NK> &w,
                                           f32x4 (&roots)[8][64], void *out, int out_bf16,
                                           int64_t M, int64_t N, int64_t r0)
{
    constexpr int LW = 1 << LWLOG;
    f32x4 stk[LWLOG > 0 ? LWLOG : 1];
    f32x4 acc;
    static_for<LW>([&](auto Jc) {
        constexpr int J = decltype(Jc)::value;
        acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, af[J * KS + kk]),
                __builtin_bit_cast(bf16x8, w.bf[J * KS + kk]), acc, 0, 0, 0);
        // binary-counter tree over the wave's leaves (lower leaves left)
        bool done = false;
#pragma unroll
        for (int b = 0; b < LWLOG; ++b) {
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
    roots[w.wave][w.lane] = acc;
    lds_barrier();
    if (w.sub == 0 && w.col < N) {
        const f32x4 *r = &roots[w.cb * S][w.lane];
        f32x4 v;
        if constexpr (S == 8)
            v = ((r[0] + r[64]) + (r[128] + r[192])) + ((r[256] + r[320]) + (r[384] + r[448]));
        else
            v = (r[0] + r[64]) + (r[128] + r[192]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int64_t row = r0 + 4 * (w.lane >> 4) + rr;
            if (row < M) {
                if (out_bf16)
                    static_cast<uint16_t *>(out)[row * N + w.col] = f32_to_bf16_rne(v[rr]);
                else
                    static_cast<float *>(out)[row * N + w.col] = v[rr];
            }
        }
    }
    lds_barrier();
}

template <int S, int LWLOG, int KS>
__global__ __launch_bounds__(512) void gemm_rows_kernel(const uint16_t *A, const uint16_t *Wt,
                                                        void *out, int out_bf16, int64_t M,
                                                        int64_t N, int64_t K)
{
    static_assert(S == 4 || S == 8, "four or eight subtrees");
    constexpr int NK = (1 << LWLOG) * KS;  // k-steps (32 columns of K) per wave
    constexpr int BPW = 8 / S;             // 16-column blocks per workgroup
    __shared__ __attribute__((aligned(16))) f32x4 roots[8][64];

    RowsWave<NK> w;
    w.lane = lane_id();
    w.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    w.sub = w.wave % S;
    w.cb = w.wave / S;
    const int64_t col0 = (static_cast<int64_t>(blockIdx.x) * BPW + w.cb) * 16;
    int64_t nb = N - col0;
    nb = nb < 0 ? 0 : (nb > 16 ? 16 : nb);
    // weight rows col0 .. col0+15; rows past N read as zero
    const __amdgpu_buffer_rsrc_t rb = tile_rsrc(Wt + (nb > 0 ? col0 : 0) * K, nb, K);
    // lane: fragment row / column (lane & 15), k-group (lane >> 4)
    w.voff = static_cast<uint32_t>((w.lane & 15) * K * 2 + (w.lane >> 4) * 16);
    w.k0 = w.sub * NK;
    w.col = col0 + (w.lane & 15);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
        w.bf[kk] = __builtin_amdgcn_raw_buffer_load_b128(rb, w.voff, (w.k0 + kk) * 64, 0);

    if (LWLOG < 3 && M > 16) {
        // 16-row groups, double-buffered: the next group's rows load while
        // the current one multiplies
        // (the loads are issued on every path, past M they read zeros
        // without touching memory: the compiler can then wait for exactly the
        // older set instead of draining every load at a branch merge)
        u32x4 a0[NK], a1[NK];
        rows_load(a0, w, A, M, K, 0);
        for (int64_t r0 = 0; r0 < M; r0 += 32) {
            rows_load(a1, w, A, M, K, r0 + 16);
            rows_group<S, LWLOG, KS>(a0, w, roots, out, out_bf16, M, N, r0);
            rows_load(a0, w, A, M, K, r0 + 32);
            if (r0 + 16 < M)
                rows_group<S, LWLOG, KS>(a1, w, roots, out, out_bf16, M, N, r0 + 16);
        }
    } else {
        // one group, or eight leaves per wave (the deeper register tree
        // leaves no room for a second row set): the groups load one after
        // the other
        u32x4 a0[NK];
        for (int64_t r0 = 0; r0 < M; r0 += 16) {
            rows_load(a0, w, A, M, K, r0);
            rows_group<S, LWLOG, KS>(a0, w, roots, out, out_bf16, M, N, r0);
        }
    }
}

template <int S, int LWLOG, int KS>
static hipError_t launch_rows(const uint16_t *A, const uint16_t *Wt, void *out, int out_bf16,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    constexpr int BPW = 8 / S;
    const int64_t blocks = (N + 16 * BPW - 1) / (16 * BPW);
    hipLaunchKernelGGL((gemm_rows_kernel<S, LWLOG, KS>), dim3(static_cast<unsigned>(blocks)),
                       dim3(512), 0, stream, A, Wt, out, out_bf16, M, N, K);
    return hipGetLastError();
}

template <int S, int LWLOG>
static hipError_t rows_ks(int ks, const uint16_t *A, const uint16_t *Wt, void *out, int out_bf16,
                          int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    constexpr int LW = 1 << LWLOG;
    switch (ks) {
    case 2: return launch_rows<S, LWLOG, 2>(A, Wt, out, out_bf16, M, N, K, stream);
    case 4:
        if constexpr (LW * 4 <= 16)
            return launch_rows<S, LWLOG, 4>(A, Wt, out, out_bf16, M, N, K, stream);
        break;
    case 8:
        if constexpr (LW * 8 <= 16)
            return launch_rows<S, LWLOG, 8>(A, Wt, out, out_bf16, M, N, K, stream);
        break;
    case 16:
        if constexpr (LW * 16 <= 16)
            return launch_rows<S, LWLOG, 16>(A, Wt, out, out_bf16, M, N, K, stream);
        break;
    default: break;
    }
    return hipErrorNotSupported;
}

hipError_t launch_gemm_rows(const uint16_t *A, const uint16_t *Wt, void *out, int out_bf16,
                            int64_t M, int64_t N, int64_t K, int leaves, int leaf_size,
                            hipStream_t stream)
{
    if (!gemm_rows_supported(M, K, leaves, leaf_size))
        return hipErrorNotSupported;
    const int ks = leaf_size / 32;
    switch (leaves) {
    case 4: return rows_ks<4, 0>(ks, A, Wt, out, out_bf16, M, N, K, stream);
    case 8: return rows_ks<8, 0>(ks, A, Wt, out, out_bf16, M, N, K, stream);
    case 16: return rows_ks<8, 1>(ks, A, Wt, out, out_bf16, M, N, K, stream);
    case 32: return rows_ks<8, 2>(ks, A, Wt, out, out_bf16, M, N, K, stream);
    case 64: return rows_ks<8, 3>(ks, A, Wt, out, out_bf16, M, N, K, stream);
    default: return hipErrorNotSupported;
    }
}

}  // namespace iso
