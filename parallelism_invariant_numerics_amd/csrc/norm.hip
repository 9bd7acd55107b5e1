// norm.hip -- batch-invariant RMSNorm with an optional residual add, for
// gfx950.
//
// Normalization is one of the reductions whose order decides a row's bits
// (katelyatop-blog post on vLLM/SkyRL IsoExec, section 4); the fix is the
// one of section 8: the contract fixes the reduction tree.  Here the sum of
// squares of a row is cut into contiguous leaves of m elements, each summed
// one term at a time in ascending order, and the leaf sums are combined by
// the balanced binary tree in leaf order.  Nothing in the schedule depends
// on the number of rows or on a row's position, and every operation is a
// correctly rounded FP32 operation, so the bits are a function of the row
// alone and a plain FP32 evaluation in the same order reproduces them.
//
// One wave per row.  Memory is accessed in row order: chunk k of lane l is
// the row's 16-byte chunk 64 k + l, so every load and store instruction of a
// wave covers 1 KiB of contiguous bytes (lanes that each held 64 or more
// contiguous bytes of their own took 20-40 % longer for rows of 2048-8192
// elements).  The sum of squares needs each leaf in one lane, so h passes
// through a wave-private LDS buffer: lane l then holds elements [l S, (l+1) S) with
// S = 8 NCH, i.e. R = S / m whole leaves (R > 1 only when the row has more
// than 64 leaves), or none when l S >= H (fewer than 64 leaves; those lanes
// add +0.0, which leaves every tree level above the real leaves unchanged).
// The lane's R leaf sums take the lowest log2 R tree levels in registers;
// the 64 lane roots take the remaining levels across lanes: partners l ^ 1,
// 2, 4, 8 by DPP row butterflies, then l ^ 16, l ^ 32.  The outputs are
// elementwise in h, the row's scale and the weight, so they are formed and
// stored in the row-order layout, from h read back from the same buffer.
#include "device_common.hpp"
#include "kernels.h"

namespace iso {

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return static_cast<uint32_t>(f32_to_bf16_rne(lo)) |
           (static_cast<uint32_t>(f32_to_bf16_rne(hi)) << 16);
}

template <int NCH, int R, bool RES>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t *__restrict__ x,
                                                      const uint16_t *res, uint16_t *res_out,
                                                      const uint16_t *__restrict__ w,
                                                      void *__restrict__ y, int out_bf16,
                                                      int64_t M, int64_t H, float eps)
{
    constexpr int S = 8 * NCH;  // elements per lane in the leaf layout
    constexpr int LM = S / R;   // leaf size
    static_assert(S % R == 0, "whole leaves per lane");
    __shared__ __attribute__((aligned(16))) u32x4 tr[4][NCH * 64];  // h of each wave's row
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wid;
    if (row >= M)
        return;  // a whole wave
    const int64_t nch = H / 8;  // 16-byte chunks in a row (64 NCH, or fewer with < 64 leaves)

    // Every load is issued unconditionally (a chunk slot past the row reads
    // chunk 0 again) and before any arithmetic, so that no branch or
    // interleaved wait separates the loads: the compiler otherwise sinks the
    // weight loads and waits between row loads (measured up to 25 % slower
    // on long rows).
    const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + row * H);
    const u32x4 *rr = reinterpret_cast<const u32x4 *>((RES ? res : x) + row * H);
    u32x4 wv[NCH];
    {
        u32x4 xv[NCH], rv[NCH];
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int64_t c = static_cast<int64_t>(k) * 64 + lane;
            const int64_t cc = c < nch ? c : 0;
            wv[k] = reinterpret_cast<const u32x4 *>(w)[cc];  // with the row, so its latency overlaps
            xv[k] = xr[cc];
            if constexpr (RES)
                rv[k] = rr[cc];
        }
        __builtin_amdgcn_sched_barrier(0);
        // h = x or bf16(x + residual), two bf16 per word, into the row's LDS
        // buffer in row order (every slot exists; slots past the row are
        // never read)
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            u32x4 hk;
            if constexpr (RES) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    hk[q] = pack_bf16(bf16_lo(xv[k][q]) + bf16_lo(rv[k][q]),
                                      bf16_hi(xv[k][q]) + bf16_hi(rv[k][q]));
            } else {
                hk = xv[k];
            }
            tr[wid][k * 64 + lane] = hk;
        }
    }
    // the LDS executes a wave's instructions in issue order; this keeps the
    // compiler from moving the reads above the writes
    __builtin_amdgcn_wave_barrier();

    // the leaf layout: lane l takes chunks l NCH .. l NCH + NCH - 1
    uint32_t h[4 * NCH];
    const bool holds = static_cast<int64_t>(lane) * S < H;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const u32x4 t = holds ? tr[wid][lane * NCH + j] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < 4; ++q)
            h[4 * j + q] = t[q];
    }

    // leaf sums (one term at a time, ascending), then the lane's subtree
    float leaf[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float s = 0.0f;
#pragma unroll
        for (int i = r * LM; i < (r + 1) * LM; ++i) {
            const float v = (i & 1) ? bf16_hi(h[i >> 1]) : bf16_lo(h[i >> 1]);
            s = s + v * v;
        }
        leaf[r] = s;
    }
#pragma unroll
    for (int width = R; width > 1; width >>= 1)
#pragma unroll
        for (int q = 0; q < width / 2; ++q)
            leaf[q] = leaf[2 * q] + leaf[2 * q + 1];
    float ss = row16_sum(leaf[0]);
    ss = ss + shfl_xor(ss, 16);
    ss = ss + shfl_xor(ss, 32);

    const float ms = ss / static_cast<float>(H);
    const float rs = 1.0f / sqrtf(ms + eps);

    // the outputs from the row-order chunks, read again from LDS (fewer live
    // registers than keeping them)
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int64_t c = static_cast<int64_t>(k) * 64 + lane;
        if (c >= nch)
            continue;
        const u32x4 hk = tr[wid][k * 64 + lane];
        if (res_out)
            reinterpret_cast<u32x4 *>(res_out + row * H)[c] = hk;
        if (out_bf16) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = pack_bf16((bf16_lo(hk[q]) * rs) * bf16_lo(wv[k][q]),
                                 (bf16_hi(hk[q]) * rs) * bf16_hi(wv[k][q]));
            reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(y) + row * H)[c] = o;
        } else {
            f32x4 *op = reinterpret_cast<f32x4 *>(static_cast<float *>(y) + row * H) + 2 * c;
#pragma unroll
            for (int q = 0; q < 4; q += 2)
                op[q / 2] = f32x4{(bf16_lo(hk[q]) * rs) * bf16_lo(wv[k][q]),
                                  (bf16_hi(hk[q]) * rs) * bf16_hi(wv[k][q]),
                                  (bf16_lo(hk[q + 1]) * rs) * bf16_lo(wv[k][q + 1]),
                                  (bf16_hi(hk[q + 1]) * rs) * bf16_hi(wv[k][q + 1])};
        }
    }
}

template <int NCH, bool RES>
static hipError_t launch_norm_r(int R, const uint16_t *x, const uint16_t *residual,
                                uint16_t *residual_out, const uint16_t *weight, void *y,
                                int out_bf16, int64_t M, int64_t H, float eps, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>((M + 3) / 4));
    switch (R) {
    case 1: hipLaunchKernelGGL((rmsnorm_kernel<NCH, 1, RES>), grid, dim3(256), 0, stream, x, residual, residual_out, weight, y, out_bf16, M, H, eps); break;
    case 2: hipLaunchKernelGGL((rmsnorm_kernel<NCH, 2, RES>), grid, dim3(256), 0, stream, x, residual, residual_out, weight, y, out_bf16, M, H, eps); break;
    case 4: hipLaunchKernelGGL((rmsnorm_kernel<NCH, 4, RES>), grid, dim3(256), 0, stream, x, residual, residual_out, weight, y, out_bf16, M, H, eps); break;
    case 8: hipLaunchKernelGGL((rmsnorm_kernel<NCH, 8, RES>), grid, dim3(256), 0, stream, x, residual, residual_out, weight, y, out_bf16, M, H, eps); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int NCH>
static hipError_t launch_norm_c(int R, const uint16_t *x, const uint16_t *residual,
                                uint16_t *residual_out, const uint16_t *weight, void *y,
                                int out_bf16, int64_t M, int64_t H, float eps, hipStream_t stream)
{
    return residual ? launch_norm_r<NCH, true>(R, x, residual, residual_out, weight, y, out_bf16, M, H, eps, stream)
                    : launch_norm_r<NCH, false>(R, x, residual, residual_out, weight, y, out_bf16, M, H, eps, stream);
}

hipError_t launch_rmsnorm(const uint16_t *x, const uint16_t *residual, uint16_t *residual_out,
                          const uint16_t *weight, void *y, int out_bf16, int64_t M, int64_t H,
                          int leaf_size, int chunks, float eps, hipStream_t stream)
{
    const int span = 8 * chunks;
    if (leaf_size <= 0 || span % leaf_size != 0)
        return hipErrorInvalidValue;
    const int R = span / leaf_size;
    switch (chunks) {
    case 1: return launch_norm_c<1>(R, x, residual, residual_out, weight, y, out_bf16, M, H, eps, stream);
    case 2: return launch_norm_c<2>(R, x, residual, residual_out, weight, y, out_bf16, M, H, eps, stream);
    case 4: return launch_norm_c<4>(R, x, residual, residual_out, weight, y, out_bf16, M, H, eps, stream);
    case 8: return launch_norm_c<8>(R, x, residual, residual_out, weight, y, out_bf16, M, H, eps, stream);
    case 16: return launch_norm_c<16>(R, x, residual, residual_out, weight, y, out_bf16, M, H, eps, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace iso
