// gemm.hip -- invariant GEMM, partition combine and the non-invariant
// comparison GEMM for gfx950.
//
// "IsoExec: Eliminating Trainer-Inference Mismatch in SkyRL" (agentlenshq),
// section "Achieving Parallelism Invariance", TP bullet: contiguous K leaves,
// FP32 accumulation, a fixed rank-to-leaf map and a fixed binary tree.  A
// partition ("emulated rank") p of P owns leaves [p L/P, (p+1) L/P); its
// workgroups write that subtree's root, and the combine kernel applies the
// top log2(P) levels of the same tree, so every P gives the same bits.
#include <atomic>
#include <type_traits>

#include "gemm_core.hpp"
#include "gemm_wide.hpp"
#include "kernels.h"

namespace iso {

int device_cus()
{
    // one entry per device; threads that race to fill an entry store the
    // same value, and the atomic keeps every read whole
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

enum OutMode : int { kOutF32 = 0, kOutBF16 = 1, kOutWorkspace = 2 };

// XCD-aware tile order: groups of kTileGroup tile columns, columns fastest
// inside a group; each XCD takes a contiguous stretch (an 8 x 8 tile block at
// 4096 x 2048), and the 32 tiles that start together on it are 8 tile
// columns x 4 tile rows.  Measured against row groups of 2-32 and column
// groups of 4 and 16 in one process, bits equal: the fastest at 4096 x 2048 x
// 2048 (8 leaves) and as fast as any at 4096^3 (16 leaves).
constexpr int kTileGroup = 8;

struct GemmParams {
    const uint16_t *A;
    const uint16_t *Wt;
    void *out;
    int64_t M, N, K;
    int64_t k_per_part;   // K columns owned by one partition
    int stages_per_leaf;  // leaf_size / 64
    int mode;             // OutMode
};

template <class C, int LOG>
__global__ __launch_bounds__(C::kThreads, 2) void gemm_leaf_kernel(GemmParams p)
{
    __shared__ __attribute__((aligned(16))) char lds[C::kLdsBytes];
    const int tm = static_cast<int>((p.M + BM - 1) / BM);
    const int tn = static_cast<int>((p.N + BN - 1) / BN);
    const int ntile = tm * tn;
    const int part = blockIdx.x / ntile;  // partition-major; tiles of a partition together
    int mt, nt;
    xcd_tile(blockIdx.x % ntile, ntile, tn, tm, kTileGroup, nt, mt);  // column groups
    const int64_t m0 = static_cast<int64_t>(mt) * BM;
    const int64_t n0 = static_cast<int64_t>(nt) * BN;

    const Pipe pipe = make_pipe<C>(p.A + m0 * p.K, p.M - m0, p.Wt + n0 * p.K, p.N - n0, p.K,
                                      part * p.k_per_part);
    Acc<C> root;
    // a wave whose rows all lie past the matrix edge (a tile of at most 64
    // rows) only keeps the ring going: its fragment reads would take LDS
    // bandwidth from the waves that have rows
    const int wr = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)) / C::WC;
    if (p.M - m0 <= static_cast<int64_t>(wr) * (BM / C::WR))
        leaf_tree_mainloop<C, LOG, true, true>(pipe, p.stages_per_leaf, lds, root);
    else
        leaf_tree_mainloop<C, LOG>(pipe, p.stages_per_leaf, lds, root);

    if (p.mode == kOutWorkspace) {
        float *ws = static_cast<float *>(p.out) + (static_cast<int64_t>(part) * p.M + m0) * p.N + n0;
        store_tile<C>(root, lds, ws, p.N, p.M - m0, p.N - n0, false);
    } else if (p.mode == kOutBF16) {
        store_tile<C>(root, lds, static_cast<uint16_t *>(p.out) + m0 * p.N + n0, p.N, p.M - m0,
                      p.N - n0, true);
    } else {
        store_tile<C>(root, lds, static_cast<float *>(p.out) + m0 * p.N + n0, p.N, p.M - m0,
                      p.N - n0, false);
    }
}

// The same contraction on 128 x 256 tiles (at most four leaves per
// workgroup, one wave per SIMD); same tile order with column groups of the
// same width in columns.
template <int LOG>
__global__ __launch_bounds__(256, 1) void gemm_wide_kernel(GemmParams p)
{
    __shared__ __attribute__((aligned(16))) char lds[kWLdsBytes];
    const int tm = static_cast<int>((p.M + BM - 1) / BM);
    const int tn = static_cast<int>((p.N + WBN - 1) / WBN);
    const int ntile = tm * tn;
    const int part = blockIdx.x / ntile;
    int mt, nt;
    xcd_tile(blockIdx.x % ntile, ntile, tn, tm, kTileGroup * BN / WBN, nt, mt);
    const int64_t m0 = static_cast<int64_t>(mt) * BM;
    const int64_t n0 = static_cast<int64_t>(nt) * WBN;
    const PipeW pipe = make_pipe_w(p.A + m0 * p.K, p.M - m0, p.Wt + n0 * p.K, p.N - n0, p.K,
                                   part * p.k_per_part);
    AccW root;
    leaf_tree_mainloop_w<LOG>(pipe, p.stages_per_leaf, lds, root);
    if (p.mode == kOutWorkspace) {
        float *ws = static_cast<float *>(p.out) + (static_cast<int64_t>(part) * p.M + m0) * p.N + n0;
        store_tile_w(root, lds, ws, p.N, p.M - m0, p.N - n0, false);
    } else if (p.mode == kOutBF16) {
        store_tile_w(root, lds, static_cast<uint16_t *>(p.out) + m0 * p.N + n0, p.N, p.M - m0,
                     p.N - n0, true);
    } else {
        store_tile_w(root, lds, static_cast<float *>(p.out) + m0 * p.N + n0, p.N, p.M - m0,
                     p.N - n0, false);
    }
}

// Top log2(P) tree levels over the partition roots ws[p][M][N].
template <int P>
__global__ __launch_bounds__(256) void partition_combine_kernel(const float *ws, void *out,
                                                                int64_t MN, int out_bf16)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < MN;
         e += stride) {
        float r[P];
#pragma unroll
        for (int q = 0; q < P; ++q)
            r[q] = ws[q * MN + e];
        const float v = fold_roots<P>(r);
        if (out_bf16)
            static_cast<uint16_t *>(out)[e] = f32_to_bf16_rne(v);
        else
            static_cast<float *>(out)[e] = v;
    }
}

// The same for four consecutive outputs per thread (16-byte loads and
// stores; MN a multiple of 4, 16-byte aligned buffers): fewer, wider memory
// requests for the small partial sets of split medium-row calls.
template <int P>
__global__ __launch_bounds__(256) void partition_combine4_kernel(const float *ws, void *out,
                                                                 int64_t MN, int out_bf16)
{
    const int64_t n4 = MN / 4;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n4;
         e += stride) {
        f32x4 r[P];
#pragma unroll
        for (int q = 0; q < P; ++q)
            r[q] = *reinterpret_cast<const f32x4 *>(ws + q * MN + 4 * e);
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float ri[P];
#pragma unroll
            for (int q = 0; q < P; ++q)
                ri[q] = r[q][i];
            v[i] = fold_roots<P>(ri);
        }
        if (out_bf16) {
            const uint32_t lo = static_cast<uint32_t>(f32_to_bf16_rne(v[0])) |
                                (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
            const uint32_t hi = static_cast<uint32_t>(f32_to_bf16_rne(v[2])) |
                                (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + 4 * e) = make_uint2(lo, hi);
        } else {
            *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + 4 * e) = v;
        }
    }
}

// The same fold, tile by tile, for roots written by gemm_leaf_kernel on a
// grid of a multiple of 8 tiles: workgroup b folds rows 8 (b / ntile) ..
// +7 of the tile that gemm_leaf_kernel's linear tile b % ntile maps to, so
// it runs on the XCD whose L2 took that tile's roots from every partition.
template <int P>
__global__ __launch_bounds__(256) void partition_combine_tiles_kernel(const float *ws, void *out,
                                                                      int64_t M, int64_t N,
                                                                      int out_bf16)
{
    const int tm = static_cast<int>((M + BM - 1) / BM);
    const int tn = static_cast<int>((N + BN - 1) / BN);
    const int ntile = tm * tn;
    int mt, nt;
    xcd_tile(blockIdx.x % ntile, ntile, tn, tm, kTileGroup, nt, mt);
    const int64_t row = static_cast<int64_t>(mt) * BM + (blockIdx.x / ntile) * 8 + (threadIdx.x >> 5);
    const int64_t col = static_cast<int64_t>(nt) * BN + 4 * (threadIdx.x & 31);
    if (row >= M || col >= N)
        return;
    const int64_t MN = M * N;
    const int64_t e = row * N + col;
    f32x4 v;
    if (col + 4 <= N) {
        f32x4 r[P];
#pragma unroll
        for (int q = 0; q < P; ++q)
            r[q] = *reinterpret_cast<const f32x4 *>(ws + q * MN + e);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float ri[P];
#pragma unroll
            for (int q = 0; q < P; ++q)
                ri[q] = r[q][i];
            v[i] = fold_roots<P>(ri);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float ri[P];
#pragma unroll
            for (int q = 0; q < P; ++q)
                ri[q] = col + i < N ? ws[q * MN + e + i] : 0.0f;
            v[i] = fold_roots<P>(ri);
        }
    }
    const int n = col + 4 <= N ? 4 : static_cast<int>(N - col);
    if (out_bf16) {
        uint16_t *o = static_cast<uint16_t *>(out) + e;
        if (n == 4) {
            const uint32_t lo = static_cast<uint32_t>(f32_to_bf16_rne(v[0])) |
                                (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
            const uint32_t hi = static_cast<uint32_t>(f32_to_bf16_rne(v[2])) |
                                (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
            *reinterpret_cast<uint2 *>(o) = make_uint2(lo, hi);
        } else {
            for (int i = 0; i < n; ++i)
                o[i] = f32_to_bf16_rne(v[i]);
        }
    } else {
        store4_f32(static_cast<float *>(out) + e, v, n == 4, n);
    }
}

hipError_t launch_partition_combine_tiles(const float *ws, void *out, int out_bf16, int64_t M,
                                          int64_t N, int parts, hipStream_t stream)
{
    const int64_t ntile = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const bool ok = ntile % kXcds == 0 && N % 4 == 0 && reinterpret_cast<uintptr_t>(ws) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(out) % (out_bf16 ? 8 : 16) == 0;
    if (!ok)
        return launch_partition_combine(ws, out, out_bf16, M * N, parts, stream);
    dim3 grid(static_cast<unsigned>(ntile * (BM / 8)));
    switch (parts) {
    case 2: hipLaunchKernelGGL(partition_combine_tiles_kernel<2>, grid, dim3(256), 0, stream, ws, out, M, N, out_bf16); break;
    case 4: hipLaunchKernelGGL(partition_combine_tiles_kernel<4>, grid, dim3(256), 0, stream, ws, out, M, N, out_bf16); break;
    case 8: hipLaunchKernelGGL(partition_combine_tiles_kernel<8>, grid, dim3(256), 0, stream, ws, out, M, N, out_bf16); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Workgroups of at most four leaves over at least 16 stages take the
// 128 x 256 tile when there is at least one such tile per CU (measured at
// 4096 x 2048 x 2048 with 4 leaves: 44.1 -> 39.7 us; 4096^3 in 4 partitions:
// 301 -> 255 us; shorter K or fewer tiles ran as fast or slower).  Otherwise
// trees of at most two leaves fit the two-workgroups-per-CU shape, which a
// grid of more workgroups than CUs fills best; deeper trees, and grids of at
// most one workgroup per CU, take the eight-wave shape (its deeper ring
// hides more of the load latency when a CU holds only one workgroup).  All
// give the same bits.
template <int LOG>
static hipError_t launch_leaf(const GemmParams &p, int parts, hipStream_t stream)
{
    if constexpr (LOG <= 2) {
        const int64_t wide = ((p.N + WBN - 1) / WBN) * ((p.M + BM - 1) / BM);
        if ((int64_t)p.stages_per_leaf << LOG >= 16 && wide * parts >= device_cus()) {
            hipLaunchKernelGGL((gemm_wide_kernel<LOG>), dim3(static_cast<unsigned>(wide * parts)),
                               dim3(256), 0, stream, p);
            return hipGetLastError();
        }
    }
    const int64_t tiles = ((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM);
    dim3 grid(static_cast<unsigned>(tiles * parts));
    if constexpr (LOG <= 1) {
        if (tiles * parts > device_cus()) {
            hipLaunchKernelGGL((gemm_leaf_kernel<CfgDual, LOG>), grid, dim3(CfgDual::kThreads), 0,
                               stream, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_leaf_kernel<CfgWide, LOG>), grid, dim3(CfgWide::kThreads), 0, stream,
                       p);
    return hipGetLastError();
}

hipError_t launch_gemm_partials(const uint16_t *A, const uint16_t *Wt, void *out, int mode,
                                int64_t M, int64_t N, int64_t K, int leaves_per_part,
                                int leaf_size, int parts, hipStream_t stream)
{
    GemmParams p;
    p.A = A;
    p.Wt = Wt;
    p.out = out;
    p.M = M;
    p.N = N;
    p.K = K;
    p.k_per_part = static_cast<int64_t>(leaves_per_part) * leaf_size;
    p.stages_per_leaf = leaf_size / BK;
    p.mode = mode;
    switch (leaves_per_part) {
    case 1: return launch_leaf<0>(p, parts, stream);
    case 2: return launch_leaf<1>(p, parts, stream);
    case 4: return launch_leaf<2>(p, parts, stream);
    case 8: return launch_leaf<3>(p, parts, stream);
    case 16: return launch_leaf<4>(p, parts, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_partition_combine(const float *ws, void *out, int out_bf16, int64_t MN, int parts,
                                    hipStream_t stream)
{
    const bool vec = MN % 4 == 0 && reinterpret_cast<uintptr_t>(ws) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(out) % (out_bf16 ? 8 : 16) == 0;
    if (vec && MN <= (int64_t)1 << 24) {  // small partial sets: latency, not bandwidth
        int64_t blocks = (MN / 4 + 255) / 256;
        if (blocks > 8192)
            blocks = 8192;
        dim3 grid(static_cast<unsigned>(blocks));
        switch (parts) {
        case 2: hipLaunchKernelGGL(partition_combine4_kernel<2>, grid, dim3(256), 0, stream, ws, out, MN, out_bf16); break;
        case 4: hipLaunchKernelGGL(partition_combine4_kernel<4>, grid, dim3(256), 0, stream, ws, out, MN, out_bf16); break;
        case 8: hipLaunchKernelGGL(partition_combine4_kernel<8>, grid, dim3(256), 0, stream, ws, out, MN, out_bf16); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    int64_t blocks = (MN + 255) / 256;
    if (blocks > 8192)
        blocks = 8192;
    dim3 grid(static_cast<unsigned>(blocks));
    switch (parts) {
    case 2: hipLaunchKernelGGL(partition_combine_kernel<2>, grid, dim3(256), 0, stream, ws, out, MN, out_bf16); break;
    case 4: hipLaunchKernelGGL(partition_combine_kernel<4>, grid, dim3(256), 0, stream, ws, out, MN, out_bf16); break;
    case 8: hipLaunchKernelGGL(partition_combine_kernel<8>, grid, dim3(256), 0, stream, ws, out, MN, out_bf16); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace iso
