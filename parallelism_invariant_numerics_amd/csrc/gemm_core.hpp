// gemm_core.hpp -- the leaf/tree contraction main loop shared by every
// kernel that computes invariant numbers (plain GEMM, LM-head, MoE experts).
//
// Numerics (one schedule for every shape): an output element's value is the
// balanced binary tree, in leaf-index order, over L leaf sums; a leaf sum
// starts at +0.0 and takes v_mfma_f32_16x16x32_bf16 steps over its K range in
// ascending order, 32 at a time.  ("IsoExec: Eliminating Trainer-Inference
// Mismatch in SkyRL", section "Achieving Parallelism Invariance", TP bullet:
// contiguous K leaves, deterministic matrix-core products with FP32
// accumulation, fixed binary tree.)  MFMA computes each output element from
// its own A row and B column only, so neither the tile shape, nor the row's
// position in the tile, nor the other rows change its bits.
//
// Tiling (gfx950): 256 threads = 4 wave64 in a 2 x 2 grid; workgroup tile
// 128 x 128; wave tile 64 x 64 = 4 x 4 MFMA blocks of 16 x 16.  K is staged
// through LDS 64 at a time (two MFMA k-steps), double buffered.  Both operands
// are k-contiguous in HBM (A [M][K], Wt [N][K]); one LDS row is the 128-byte
// k-slice of one matrix row, its eight 16-byte chunks XOR-swizzled by
// (row & 7) so that the MFMA fragment reads (16 rows x one chunk) and the
// staging writes (8 rows x 8 chunks) spread over all banks.
//
// The tree over the leaves of one workgroup is kept in registers as a
// binary-counter stack: after leaf J, the running value absorbs the saved
// left sibling at every level where bit b of J is 1, and is saved at the
// first level where it is 0.  Depth log2(leaves) + 1 accumulator sets.
#pragma once

#include <utility>

#include "device_common.hpp"

namespace iso {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kRowBytes = BK * 2;                        // 128 bytes per LDS row
constexpr int kStageBytes = (BM + BN) * kRowBytes;        // 32 KiB per stage
constexpr int kLdsBytes = 2 * kStageBytes;                // 64 KiB, double buffered
constexpr int kMaxLogLeavesPerTile = 4;                   // register stack depth bound

struct Acc {
    f32x4 v[4][4];
};

__device__ __forceinline__ void acc_zero(Acc &a)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            a.v[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// dst = left + right, element by element (one FP32 add, round to nearest).
__device__ __forceinline__ void acc_add(Acc &dst, const Acc &left, const Acc &right)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            dst.v[i][j] = left.v[i][j] + right.v[i][j];
}

// Fold one finished leaf (index J within the tile's leaf block) into the
// register tree.  After the last leaf, `v` holds the block's subtree root.
template <int LOG, int J, int B>
__device__ __forceinline__ void tree_push(Acc (&stk)[LOG > 0 ? LOG : 1], Acc &v)
{
    if constexpr (B < LOG) {
        if constexpr (((J >> B) & 1) != 0) {
            acc_add(v, stk[B], v);  // left sibling (lower leaf indices) + right
            tree_push<LOG, J, B + 1>(stk, v);
        } else {
            stk[B] = v;
        }
    }
}

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}

template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(static_cast<F &&>(f), std::make_integer_sequence<int, N>{});
}

// Per-thread global sources: this thread stages rows (tid/8 + 32 i), i < 4,
// of both operand tiles, 16-byte chunk (tid & 7) of each 64-wide k-slice.
// Pointers already include the chunk offset and the tile's first k.
struct TileSrc {
    const uint16_t *a[4];
    const uint16_t *b[4];
};

struct StageRegs {
    u32x4 a[4];
    u32x4 b[4];
};

__device__ __forceinline__ void stage_load(StageRegs &r, const TileSrc &src, int64_t k)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r.a[i] = *reinterpret_cast<const u32x4 *>(src.a[i] + k);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r.b[i] = *reinterpret_cast<const u32x4 *>(src.b[i] + k);
}

__device__ __forceinline__ void stage_store(const StageRegs &r, char *stage, int tid)
{
    const int c = tid & 7;
    const int sw = ((c ^ ((tid >> 3) & 7)) << 4);
    char *As = stage;
    char *Bs = stage + BM * kRowBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 3) + 32 * i;
        *reinterpret_cast<u32x4 *>(As + row * kRowBytes + sw) = r.a[i];
        *reinterpret_cast<u32x4 *>(Bs + row * kRowBytes + sw) = r.b[i];
    }
}

// Two MFMA k-steps (k 0..31, then 32..63 of the stage) into acc.
__device__ __forceinline__ void stage_mfma(Acc &acc, const char *stage, int lane, int wr, int wc)
{
    const char *As = stage + (wr * 64 + (lane & 15)) * kRowBytes;
    const char *Bs = stage + BM * kRowBytes + (wc * 64 + (lane & 15)) * kRowBytes;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int chunk = (((s * 4) + (lane >> 4)) ^ (lane & 7)) << 4;
        bf16x8 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = *reinterpret_cast<const bf16x8 *>(As + i * 16 * kRowBytes + chunk);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[j] = *reinterpret_cast<const bf16x8 *>(Bs + j * 16 * kRowBytes + chunk);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc.v[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc.v[i][j], 0,
                                                                      0, 0);
    }
}

// The contraction of one tile over 2^LOG leaves of `stages_per_leaf` * 64
// columns of K each.  On return `root` holds the subtree root in the MFMA
// output layout; every thread has passed a final barrier, so `lds` may be
// reused by the caller.
template <int LOG>
__device__ __forceinline__ void leaf_tree_mainloop(const TileSrc &src, int stages_per_leaf,
                                                   char *lds, Acc &root)
{
    constexpr int LP = 1 << LOG;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave >> 1;
    const int wc = wave & 1;
    const int nst = LP * stages_per_leaf;

    StageRegs regs;
    stage_load(regs, src, 0);
    stage_store(regs, lds, tid);
    __syncthreads();

    Acc stk[LOG > 0 ? LOG : 1];
    Acc acc;
    int st = 0;
    static_for<LP>([&](auto J) {
        acc_zero(acc);
        for (int s = 0; s < stages_per_leaf; ++s, ++st) {
            const bool more = st + 1 < nst;
            if (more)
                stage_load(regs, src, static_cast<int64_t>(st + 1) * BK);
            stage_mfma(acc, lds + (st & 1) * kStageBytes, lane, wr, wc);
            if (more)
                stage_store(regs, lds + ((st + 1) & 1) * kStageBytes, tid);
            __syncthreads();
        }
        tree_push<LOG, decltype(J)::value, 0>(stk, acc);
        if constexpr (decltype(J)::value == LP - 1)
            root = acc;
    });
}

// Row and column (within the 128 x 128 tile) of acc.v[i][j][r] for this lane.
__device__ __forceinline__ int tile_row(int lane, int wr, int i, int r)
{
    return wr * 64 + i * 16 + (lane >> 4) * 4 + r;
}
__device__ __forceinline__ int tile_col(int lane, int wc, int j)
{
    return wc * 64 + j * 16 + (lane & 15);
}

// Fixed tree over P partition roots (P = 1, 2, 4, 8), lower index left.
template <int P>
__device__ __forceinline__ float fold_roots(const float (&r)[P])
{
    if constexpr (P == 1) {
        return r[0];
    } else if constexpr (P == 2) {
        return r[0] + r[1];
    } else if constexpr (P == 4) {
        return (r[0] + r[1]) + (r[2] + r[3]);
    } else {
        static_assert(P == 8, "partition counts are 1, 2, 4, 8");
        return ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
    }
}

}  // namespace iso
