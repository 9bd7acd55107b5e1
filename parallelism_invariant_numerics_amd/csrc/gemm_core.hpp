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
// its own A row and B column only, so neither the tile shape, nor the wave
// layout, nor the row's position in the tile, nor the other rows change its
// bits: the two launch shapes below give identical results.
//
// Tiling (gfx950): a workgroup computes a 128 x 128 output tile with its
// waves in a 2 x WC grid (wave tile 64 x 128/WC, built from 16 x 16 MFMA
// blocks).  Both operands are k-contiguous in HBM (A [M][K], Wt [N][K]).  K
// moves through LDS 64 at a time ("stages") in a ring of 32 KiB stage buffers
// filled by direct global-to-LDS buffer loads issued NBUF-1 stages ahead, so
// no staging registers are needed.  One LDS row holds the 128-byte k-slice of
// one matrix row; its eight 16-byte chunks are XOR-swizzled by (row & 7),
// which keeps the 16-row fragment reads free of bank conflicts.  Rows past
// the matrix edge read as zero (buffer range check) and are never stored.
//
// Launch shapes (both keep two waves on every SIMD, which the MFMA pipe needs
// to stay busy across LDS and barrier waits):
//   CfgWide: 8 waves (2 x 4, wave tile 64 x 32), one workgroup per CU, a
//            four-stage ring (128 KiB).  Holds a 3- or 4-level register tree.
//   CfgDual: 4 waves (2 x 2, wave tile 64 x 64), two workgroups per CU, a
//            two-stage ring (64 KiB).  Register room for at most one tree
//            level; the second workgroup hides the first one's waits.
//
// Fragment reads are issued ahead of the MFMAs that use them: the second
// k-step's fragments of a stage load while the first k-step multiplies, and
// the first k-step of the next stage loads while the previous stage's second
// k-step multiplies.  The LDS reads and the waits are inline assembly so that
// the compiler does not add conservative waits for the in-flight global-to-LDS
// loads of later stages.
//
// The tree over the leaves of one workgroup is kept in registers as a
// binary-counter stack: after leaf J, the running value absorbs the saved
// left sibling at every level where bit b of J is 1, and is saved at the
// first level where it is 0.  Saved sums are parked in AGPRs.
#pragma once

#include <utility>

#include "device_common.hpp"

#define ISO_LDS __attribute__((address_space(3)))

namespace iso {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kRowBytes = BK * 2;                    // 128 bytes per LDS row
constexpr int kStageBytes = (BM + BN) * kRowBytes;   // 32 KiB per stage
constexpr int kBOffset = BM * kRowBytes;             // B tile inside a stage

template <int WC_, int NBUF_>
struct TileCfg {
    static constexpr int WR = 2;
    static constexpr int WC = WC_;
    static constexpr int kWaves = WR * WC;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int IB = BM / WR / 16;  // 16-row blocks per wave
    static constexpr int JB = BN / WC / 16;  // 16-column blocks per wave
    static constexpr int NBUF = NBUF_;
    static constexpr int kLdsBytes = NBUF * kStageBytes;
    static constexpr int kDma = BM / kWaves / 8;  // buffer loads per operand per wave per stage
};
using CfgWide = TileCfg<4, 4>;
using CfgDual = TileCfg<2, 2>;

template <class C>
struct Acc {
    f32x4 v[C::IB][C::JB];
};

// One 32-deep MFMA k-step's operands: A row blocks i and B column blocks j.
template <class C>
struct Frags {
    bf16x8 a[C::IB];
    bf16x8 b[C::JB];
};

template <class C>
__device__ __forceinline__ void acc_zero(Acc<C> &a)
{
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
#pragma unroll
        for (int j = 0; j < C::JB; ++j)
            a.v[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

template <class C>
__device__ __forceinline__ void mfma_step(Acc<C> &acc, const Frags<C> &f)
{
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
#pragma unroll
        for (int j = 0; j < C::JB; ++j)
            acc.v[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc.v[i][j], 0,
                                                                  0, 0);
}

// Saved subtree sums are parked in the accumulation registers (AGPRs); these
// empty asm statements only pin the register class (values pass unchanged).
template <class C>
__device__ __forceinline__ void park(Acc<C> &dst, const Acc<C> &src)
{
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
#pragma unroll
        for (int j = 0; j < C::JB; ++j) {
            f32x4 t = src.v[i][j];
            asm volatile("" : "=a"(t) : "0"(t));
            dst.v[i][j] = t;
        }
}

// v = left + v element by element (left sibling = lower leaf indices).
template <class C>
__device__ __forceinline__ void unpark_add(Acc<C> &v, const Acc<C> &left)
{
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
#pragma unroll
        for (int j = 0; j < C::JB; ++j) {
            f32x4 t = left.v[i][j];
            asm volatile("" : "=v"(t) : "0"(t));
            v.v[i][j] = t + v.v[i][j];
        }
}

// Fold one finished leaf (index J within the tile's leaf block) into the
// register tree.  After the last leaf, `v` holds the block's subtree root.
template <class C, int LOG, int J, int B>
__device__ __forceinline__ void tree_push(Acc<C> (&stk)[LOG > 0 ? LOG : 1], Acc<C> &v)
{
    if constexpr (B < LOG) {
        if constexpr (((J >> B) & 1) != 0) {
            unpark_add(v, stk[B]);
            tree_push<C, LOG, J, B + 1>(stk, v);
        } else {
            park(stk[B], v);
        }
    }
}

// This lane's index in its wave, as a value the compiler must recompute
// where it is used: persistent kernels loop over tiles, and hoisting every
// lane-derived address out of that loop costs more registers than it saves.
__device__ __forceinline__ int lane_id()
{
    int l = static_cast<int>(threadIdx.x & 63);
    asm volatile("" : "+v"(l));
    return l;
}

// ------------------------------------------------------------------ sources

// A 128-row operand tile: rows [0, rows) of a k-contiguous matrix starting at
// `base`, `K` elements per row.  Rows at or past `rows` read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *base, int64_t rows,
                                                            int64_t K)
{
    int64_t bytes = rows * K * 2;
    if (bytes > 0xffffffffLL)
        bytes = 0xffffffffLL;
    if (bytes < 0)
        bytes = 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), (short)0,
                                             (int)(uint32_t)bytes, 0x00020000);
}

// Per-thread state of the stage pipeline of one tile (kDma <= 4 entries of
// voff are used).
constexpr int kMaxDma = 4;
struct Pipe {
    __amdgpu_buffer_rsrc_t ra, rb;  // A rows, B tile rows
    uint32_t voffa[kMaxDma];        // this lane's byte offsets for its A and B DMA rows
    uint32_t voffb[kMaxDma];
    uint32_t kbyte0;                // byte offset of the tile's first k (partition start)
};

// Lane l of wave w stages, for i < kDma, row r = kDma*8 w + 8 i + (l >> 3)
// and the global 16-byte chunk c = (l & 7) ^ (r & 7) into LDS slot (r, l & 7)
// of both the A and the B tile: one buffer load fills 8 consecutive LDS rows,
// 1 KiB, lane by lane.  A rows [rowsA, 128) and B rows [rowsB, 128) are past
// the matrix edge and read as zero.
template <class C>
__device__ __forceinline__ Pipe make_pipe(const uint16_t *A_tile, int64_t rowsA,
                                             const uint16_t *B_tile, int64_t rowsB, int64_t K,
                                             int64_t k0)
{
    static_assert(C::kDma <= kMaxDma, "too many loads per wave");
    Pipe p;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    p.ra = tile_rsrc(A_tile, rowsA < BM ? rowsA : BM, K);
    p.rb = tile_rsrc(B_tile, rowsB < BN ? rowsB : BN, K);
    const uint32_t c = (lane & 7) ^ (lane >> 3);
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) {
        const uint32_t r = C::kDma * 8 * w + 8 * i + (lane >> 3);
        p.voffa[i] = (uint32_t)((int64_t)r * K * 2) + c * 16;
        p.voffb[i] = p.voffa[i];
    }
    p.kbyte0 = (uint32_t)(k0 * 2);
    return p;
}

template <class C>
__device__ __forceinline__ void stage_dma(const Pipe &p, char *lds, int st, int buf)
{
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t soff = p.kbyte0 + (uint32_t)st * (BK * 2);
    char *dst = lds + buf * kStageBytes + w * C::kDma * 8 * kRowBytes;
#pragma unroll
    for (int i = 0; i < C::kDma; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(p.ra, (ISO_LDS void *)(dst + i * 8 * kRowBytes),
                                                 16, p.voffa[i], soff, 0, 0);
#pragma unroll
    for (int i = 0; i < C::kDma; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            p.rb, (ISO_LDS void *)(dst + kBOffset + i * 8 * kRowBytes), 16, p.voffb[i], soff, 0,
            0);
}

// Wait until at most `pending` later stages of this wave's buffer loads
// (2 kDma loads per stage) are still in flight, then synchronise the
// workgroup.  The count n is the number of loads this wave issued after the
// awaited stage.  Loads complete in order, so while any load of that stage
// is outstanding all n later loads are too: at least n + 1 operations are
// in flight, whatever stores (epilogue writes, register spills) do, and the
// wait cannot pass early.
template <class C>
__device__ __forceinline__ void stage_barrier(int pending)
{
    constexpr int D = 2 * C::kDma;
    if (pending >= 2)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * D) : "memory");
    else if (pending == 1)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(D) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

// Issue the LDS reads of one k-step's fragments (no wait).
template <class C>
__device__ __forceinline__ void frag_read(Frags<C> &f, uint32_t addr_a, uint32_t addr_b)
{
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
        asm volatile("ds_read_b128 %0, %1 offset:%2"
                     : "=&v"(f.a[i])
                     : "v"(addr_a), "n"(i * 16 * kRowBytes));
#pragma unroll
    for (int j = 0; j < C::JB; ++j)
        asm volatile("ds_read_b128 %0, %1 offset:%2"
                     : "=&v"(f.b[j])
                     : "v"(addr_b), "n"(j * 16 * kRowBytes));
}

// Wait for all LDS reads of this wave; the fragments become usable after it.
template <class C>
__device__ __forceinline__ void frag_wait(Frags<C> &f)
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
        asm volatile("" : "+v"(f.a[i]));
#pragma unroll
    for (int j = 0; j < C::JB; ++j)
        asm volatile("" : "+v"(f.b[j]));
}

// First NBUF-1 stages of a tile's ring (`nst` stages in all).  A persistent
// kernel issues them for its next tile as soon as the current tile's main
// loop has returned, so that their latency overlaps the epilogue.
template <class C>
__device__ __forceinline__ void pipe_prologue(const Pipe &p, char *lds, int nst)
{
#pragma unroll
    for (int s = 0; s < C::NBUF - 1; ++s)
        if (s < nst)
            stage_dma<C>(p, lds, s, s);
}

// The contraction of one tile over 2^LOG leaves of `spl` stages (64 columns
// of K) each.  With PROLOGUE false the caller has already issued
// pipe_prologue for this tile (and nothing else on the ring since).  On
// return `root` holds the subtree root in the MFMA output layout, every
// buffer load has landed and all waves have passed a final barrier, so `lds`
// may be reused by the caller.  Global stores or loads that the caller has in
// flight only make the ring's vmcnt waits stricter (loads complete in order,
// so "at most n outstanding" still implies that the oldest stage landed).
//
// A buffer load holds up the wave that issues it until the address unit has
// taken it, and that unit is shared by the CU.  Waves w and w + 4 of an
// eight-wave workgroup share a SIMD, so the upper four waves issue their
// loads of the stage after their first k-step's MFMAs instead of right after
// the barrier: while one wave of a SIMD waits on the address unit, the other
// one keeps the matrix core busy.  The loads still go out before the next
// stage's wait, so the ring's counts are unchanged.
// With IDLE the wave owns no row of the tile (all of its rows lie past the
// matrix edge): it issues exactly the ring loads and barriers of the other
// waves, in the same order, and no fragment read or MFMA, so the stage ring
// keeps its counts while the LDS serves only the waves with rows; `root` is
// zero and never stored.
template <class C, int LOG, bool PROLOGUE = true, bool IDLE = false>
__device__ __forceinline__ void leaf_tree_mainloop(const Pipe &p, int spl, char *lds,
                                                   Acc<C> &root)
{
    constexpr int LP = 1 << LOG;
    constexpr int NB = C::NBUF;
    const int nst = LP * spl;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / C::WC;
    const int wc = wave % C::WC;
    const bool late = C::kWaves == 8 && wave >= 4;

    const uint32_t lds_addr = (uint32_t)(uintptr_t)(ISO_LDS char *)lds;
    const uint32_t ch0 = (uint32_t)(((lane >> 4) ^ (lane & 7)) << 4);
    const uint32_t ch1 = ch0 ^ 64u;  // chunks 4..7 of the row: second k-step
    const uint32_t rowa = (uint32_t)(wr * (BM / C::WR) + (lane & 15)) * kRowBytes;
    const uint32_t rowb =
        (uint32_t)kBOffset + (uint32_t)(wc * (BN / C::WC) + (lane & 15)) * kRowBytes;

    if constexpr (PROLOGUE)
        pipe_prologue<C>(p, lds, nst);

    if constexpr (IDLE) {
        for (int st = 0; st < nst; ++st) {
            const int ahead = nst - 1 - st;
            stage_barrier<C>(ahead < NB - 2 ? ahead : NB - 2);
            if (st + NB - 1 < nst)
                stage_dma<C>(p, lds, st + NB - 1, (st + NB - 1) % NB);
        }
        acc_zero(root);
        __builtin_amdgcn_s_barrier();
        return;
    }

    Acc<C> stk[LOG > 0 ? LOG : 1];
    Acc<C> acc;
    acc_zero(acc);
    Frags<C> f0, f1;
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
        f1.a[i] = bf16x8{};
#pragma unroll
    for (int j = 0; j < C::JB; ++j)
        f1.b[j] = bf16x8{};
    int st = 0;
    static_for<LP>([&](auto Jc) {
        constexpr int J = decltype(Jc)::value;
        for (int s = 0; s < spl; ++s, ++st) {
            frag_wait(f1);  // previous stage's reads done before its buffer is recycled
            const int ahead = nst - 1 - st;
            stage_barrier<C>(ahead < NB - 2 ? ahead : NB - 2);
            const bool dma = st + NB - 1 < nst;
            if (dma && !late)
                stage_dma<C>(p, lds, st + NB - 1, (st + NB - 1) % NB);
            const uint32_t base = lds_addr + (uint32_t)(st % NB) * kStageBytes;
            frag_read(f0, base + rowa + ch0, base + rowb + ch0);
            if (st > 0) {
                mfma_step(acc, f1);  // second k-step of the previous stage
                if constexpr (J > 0) {
                    if (s == 0) {  // the previous stage closed leaf J - 1
                        tree_push<C, LOG, J - 1, 0>(stk, acc);
                        acc_zero(acc);
                    }
                }
            }
            if (dma && late)
                stage_dma<C>(p, lds, st + NB - 1, (st + NB - 1) % NB);
            frag_wait(f0);
            frag_read(f1, base + rowa + ch1, base + rowb + ch1);
            mfma_step(acc, f0);
        }
    });
    frag_wait(f1);
    mfma_step(acc, f1);
    tree_push<C, LOG, LP - 1, 0>(stk, acc);
    root = acc;
    __builtin_amdgcn_s_barrier();
}

// Row and column (within the 128 x 128 tile) of acc.v[i][j][r] for this lane.
template <class C>
__device__ __forceinline__ int tile_row(int lane, int wr, int i, int r)
{
    return wr * (BM / C::WR) + i * 16 + (lane >> 4) * 4 + r;
}
template <class C>
__device__ __forceinline__ int tile_col(int lane, int wc, int j)
{
    return wc * (BN / C::WC) + j * 16 + (lane & 15);
}

// ------------------------------------------------------------------ epilogue

// A tile's FP32 roots staged in LDS so that the global stores can be whole
// 16-byte vectors instead of one element per lane; the values pass unchanged.
// Layout: 128 rows of 512 bytes; the 16-byte chunk c of row r sits at chunk
// c ^ (4 ((r >> 2) & 3)), which puts the four row groups of one MFMA output
// register on disjoint banks.  `lds` must hold 64 KiB that no wave still
// reads (the stage ring after leaf_tree_mainloop returns); the function ends
// with a workgroup barrier.
template <class C>
__device__ __forceinline__ const float *stage_tile(const Acc<C> &root, char *lds)
{
    static_assert(C::kLdsBytes >= BM * BN * 4, "the stage ring must hold the FP32 tile");
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave / C::WC, wc = wave % C::WC;
    float *stage = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
#pragma unroll
        for (int j = 0; j < C::JB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = tile_row<C>(lane, wr, i, r);
                const int col = tile_col<C>(lane, wc, j);
                const int chunk = (col >> 2) ^ (((row >> 2) & 3) << 2);
                stage[row * 128 + chunk * 4 + (col & 3)] = root.v[i][j][r];
            }
    __syncthreads();
    return stage;
}

// Columns 4c .. 4c+3 of staged row `row`.
__device__ __forceinline__ f32x4 staged_chunk(const float *stage, int row, int c)
{
    return *reinterpret_cast<const f32x4 *>(stage + row * 128 +
                                            ((c ^ (((row >> 2) & 3) << 2)) << 2));
}

// Store 8 bf16 (rounded to nearest even) or 4 FP32 values at dst, whole when
// `vec` (16-byte aligned and all in range), else only the first `n`.
__device__ __forceinline__ void store8_bf16(uint16_t *dst, const float (&v)[8], bool vec, int n)
{
    if (vec) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = static_cast<uint32_t>(f32_to_bf16_rne(v[2 * e])) |
                   (static_cast<uint32_t>(f32_to_bf16_rne(v[2 * e + 1])) << 16);
        *reinterpret_cast<u32x4 *>(dst) = w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < n)
                dst[e] = f32_to_bf16_rne(v[e]);
    }
}
__device__ __forceinline__ void store4_f32(float *dst, const f32x4 &v, bool vec, int n)
{
    if (vec) {
        *reinterpret_cast<f32x4 *>(dst) = v;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < n)
                dst[e] = v[e];
    }
}

// Write a tile's roots to a row-major output: FP32 unchanged or bf16 rounded
// to nearest even.  Tile row r goes to output row r, or to row_map[r] when
// `row_map` is given.
//   out       tile column 0 of output row 0
//   ld        output row stride in elements
//   rows, cols  rows / columns of the tile inside the matrix (clipped to 128)
template <class C>
__device__ __forceinline__ void store_tile(const Acc<C> &root, char *lds, void *out, int64_t ld,
                                           int64_t rows, int64_t cols, bool bf16_out,
                                           const int32_t *row_map = nullptr)
{
    const float *stage = stage_tile<C>(root, lds);
    const int rmax = rows < BM ? static_cast<int>(rows) : BM;
    const int cmax = cols < BN ? static_cast<int>(cols) : BN;
    if (bf16_out) {
        uint16_t *o = static_cast<uint16_t *>(out);
        const bool al = (reinterpret_cast<uintptr_t>(o) % 16 == 0) && (ld % 8 == 0);
        for (int u = threadIdx.x; u < BM * 16; u += C::kThreads) {
            const int row = u >> 4, q = u & 15;
            if (row >= rmax)
                break;
            const f32x4 lo = staged_chunk(stage, row, 2 * q);
            const f32x4 hi = staged_chunk(stage, row, 2 * q + 1);
            const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const int64_t orow = row_map ? row_map[row] : row;
            store8_bf16(o + orow * ld + 8 * q, v, al && 8 * q + 8 <= cmax, cmax - 8 * q);
        }
    } else {
        float *o = static_cast<float *>(out);
        const bool al = (reinterpret_cast<uintptr_t>(o) % 16 == 0) && (ld % 4 == 0);
        for (int u = threadIdx.x; u < BM * 32; u += C::kThreads) {
            const int row = u >> 5, q = u & 31;
            if (row >= rmax)
                break;
            const int64_t orow = row_map ? row_map[row] : row;
            store4_f32(o + orow * ld + 4 * q, staged_chunk(stage, row, q), al && 4 * q + 4 <= cmax,
                       cmax - 4 * q);
        }
    }
}

// XCD-aware tile order.  Workgroups are dispatched round-robin over the
// 8 XCDs (workgroup b runs on XCD b % 8), and each XCD has its own L2.  The
// linear workgroup id is renumbered so that each XCD walks one contiguous
// stretch of a grouped tile order (G tile rows at a time, rows fastest),
// i.e. a compact block of output tiles whose A rows and B columns its L2
// shares.  Returns the tile's (row block, column block) in a tm x tn grid.
constexpr int kXcds = 8;

// Tile t of the grouped order: G tile rows at a time, rows fastest.
__device__ __forceinline__ void grouped_tile(int t, int tm, int tn, int group, int &mt, int &nt)
{
    const int gsz_full = group * tn;
    const int g = t / gsz_full;
    const int first = g * group;
    const int rows = tm - first < group ? tm - first : group;
    const int r = t % gsz_full;
    mt = first + r % rows;
    nt = r / rows;
}

__device__ __forceinline__ void xcd_tile(int bid, int nblocks, int tm, int tn, int group,
                                         int &mt, int &nt)
{
    const int xcd = bid % kXcds;
    const int per = nblocks / kXcds;
    const int extra = nblocks % kXcds;
    const int t = xcd * per + (xcd < extra ? xcd : extra) + bid / kXcds;
    grouped_tile(t, tm, tn, group, mt, nt);
}

// LDS access in inline assembly, for code that runs while direct
// global-to-LDS loads are in flight: the compiler would otherwise make every
// LDS access there wait for them (it cannot tell the buffers apart).  Reads
// are issued, then lds_wait() completes them and pins the results, so that
// no use is scheduled before the wait.  The compiler still takes a read's
// output as written when the asm statement ends, so under register pressure
// it may copy or spill it before the wait; the CPU test suite scans the
// assembly of every kernel for that, and where it happens the reads and their
// wait go into one asm statement instead.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(ISO_LDS const char *)p;
}
__device__ __forceinline__ void lds_write_f32(uint32_t addr, float v)
{
    asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_issue_b128(f32x4 &v, uint32_t addr)
{
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
}
__device__ __forceinline__ void lds_issue_b32(int32_t &v, uint32_t addr)
{
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
}
__device__ __forceinline__ void lds_wait()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}
template <class T>
__device__ __forceinline__ void lds_pin(T &v)
{
    asm volatile("" : "+v"(v));
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
