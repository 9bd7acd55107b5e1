// gemm_rows.hip -- the leaf/tree GEMM for calls of at most 32 rows (decode
// steps of a linear layer), for gfx950.
//
// Numerics: those of gemm_core.hpp ("IsoExec: Eliminating Trainer-Inference
// Mismatch in SkyRL", section "Achieving Parallelism Invariance", TP bullet:
// contiguous K leaves, FP32 accumulation, one fixed binary tree).  Each leaf
// sum is the same chain of v_mfma_f32_16x16x32_bf16 steps in ascending k,
// started from +0.0, and the leaves are combined by the same balanced tree,
// so an element has the bits the tile kernels give it in any batch.
//
// Why a kernel of its own: with one to 32 rows the work is the weight
// stream (N x K bf16), and a 128 x 128 output tile per workgroup leaves all
// but N / 128 CUs idle.  Here a workgroup of eight waves takes 16 output
// columns (two blocks of 16 for four leaves); wave w of a block takes the
// contiguous subtree of L / S leaves number w (S = 8, or 4 for four
// leaves), loads all of its weight and row fragments into registers at once,
// and folds its leaves with the register tree, one accumulator per 16-row
// MFMA block (two above 16 rows).  The S subtree roots meet in LDS, where the
// top log2 S tree levels combine them in index order.
#include "gemm_core.hpp"
#include "kernels.h"

namespace iso {

constexpr int kRowsMax = 32;  // two 16-row MFMA blocks
constexpr int64_t kRowsMaxK = 4096;

template <int S, int LWLOG, int KS, int RB>
__global__ __launch_bounds__(512) void gemm_rows_kernel(const uint16_t *A, const uint16_t *Wt,
                                                        void *out, int out_bf16, int64_t M,
                                                        int64_t N, int64_t K)
{
    static_assert(S == 4 || S == 8, "four or eight subtrees");
    constexpr int LW = 1 << LWLOG;  // leaves per wave
    constexpr int NK = LW * KS;     // k-steps (32 columns of K) per wave
    constexpr int BPW = 8 / S;      // 16-column blocks per workgroup
    __shared__ __attribute__((aligned(16))) f32x4 roots[RB][8][64];

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = wave % S;
    const int cb = wave / S;
    const int64_t col0 = (static_cast<int64_t>(blockIdx.x) * BPW + cb) * 16;
    int64_t nb = N - col0;
    nb = nb < 0 ? 0 : (nb > 16 ? 16 : nb);
    // weight rows col0 .. col0+15 and the call's rows; rows past N or M read as zero
    const __amdgpu_buffer_rsrc_t rb = tile_rsrc(Wt + (nb > 0 ? col0 : 0) * K, nb, K);
    const __amdgpu_buffer_rsrc_t ra = tile_rsrc(A, M, K);
    // lane: fragment row / column (lane & 15), k-group (lane >> 4)
    const uint32_t voff = static_cast<uint32_t>((lane & 15) * K * 2 + (lane >> 4) * 16);
    const int k0 = sub * NK;

    u32x4 af[RB][NK], bf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
        bf[kk] = __builtin_amdgcn_raw_buffer_load_b128(rb, voff, (k0 + kk) * 64, 0);
#pragma unroll
        for (int q = 0; q < RB; ++q)  // row block q: rows 16 q .. 16 q + 15
            af[q][kk] = __builtin_amdgcn_raw_buffer_load_b128(
                ra, voff + static_cast<uint32_t>(16 * q * K * 2), (k0 + kk) * 64, 0);
    }

    f32x4 stk[RB][LWLOG > 0 ? LWLOG : 1];
    f32x4 acc[RB];
    static_for<LW>([&](auto Jc) {
        constexpr int J = decltype(Jc)::value;
#pragma unroll
        for (int q = 0; q < RB; ++q) {
            acc[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, af[q][J * KS + kk]),
                    __builtin_bit_cast(bf16x8, bf[J * KS + kk]), acc[q], 0, 0, 0);
            // binary-counter tree over the wave's leaves (lower leaves left)
            bool done = false;
#pragma unroll
            for (int b = 0; b < LWLOG; ++b) {
                if (!done) {
                    if ((J >> b) & 1) {
                        acc[q] = stk[q][b] + acc[q];
                    } else {
                        stk[q][b] = acc[q];
                        done = true;
                    }
                }
            }
        }
    });

#pragma unroll
    for (int q = 0; q < RB; ++q)
        roots[q][wave][lane] = acc[q];
    __syncthreads();
    if (sub != 0)
        return;
    const int64_t col = col0 + (lane & 15);
    if (col >= N)
        return;
#pragma unroll
    for (int q = 0; q < RB; ++q) {
        const f32x4 *r = &roots[q][cb * S][lane];
        f32x4 v;
        if constexpr (S == 8)
            v = ((r[0] + r[64]) + (r[128] + r[192])) + ((r[256] + r[320]) + (r[384] + r[448]));
        else
            v = (r[0] + r[64]) + (r[128] + r[192]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int64_t row = 16 * q + 4 * (lane >> 4) + rr;
            if (row < M) {
                if (out_bf16)
                    static_cast<uint16_t *>(out)[row * N + col] = f32_to_bf16_rne(v[rr]);
                else
                    static_cast<float *>(out)[row * N + col] = v[rr];
            }
        }
    }
}

template <int S, int LWLOG, int KS>
static hipError_t launch_rows(const uint16_t *A, const uint16_t *Wt, void *out, int out_bf16,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    constexpr int BPW = 8 / S;
    const int64_t blocks = (N + 16 * BPW - 1) / (16 * BPW);
    if (M <= 16)
        hipLaunchKernelGGL((gemm_rows_kernel<S, LWLOG, KS, 1>), dim3(static_cast<unsigned>(blocks)),
                           dim3(512), 0, stream, A, Wt, out, out_bf16, M, N, K);
    else
        hipLaunchKernelGGL((gemm_rows_kernel<S, LWLOG, KS, 2>), dim3(static_cast<unsigned>(blocks)),
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
    if (M < 1 || M > kRowsMax || K > kRowsMaxK || leaf_size % 32 != 0)
        return hipErrorNotSupported;
    const int ks = leaf_size / 32;
    if (static_cast<int64_t>(ks) * 32 * leaves != K)
        return hipErrorNotSupported;
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
