// gemm_wide.hpp -- the leaf/tree main loop on a 128 x 256 output tile, for
// workgroups that hold at most four leaves.
//
// Numerics: identical to gemm_core.hpp (the schedule is the definition):
// every leaf sum starts at +0.0 and takes v_mfma_f32_16x16x32_bf16 steps over
// its K range in ascending order, and the leaf sums of the workgroup go
// through the same balanced binary-counter tree.  MFMA computes each output
// element from its own A row and B column only, so the wider tile, the wave
// layout and the instruction order give the same bits as the 128 x 128
// kernels.  ("IsoExec: Eliminating Trainer-Inference Mismatch in SkyRL",
// section "Achieving Parallelism Invariance", TP bullet.)
//
// Why a wider tile: the 128 x 128 loop is held by its memory instructions
// (one 1 KiB global-to-LDS load per 8 MFMAs and 0.5-0.75 fragment reads per
// MFMA), not by waiting on data.  A 128 x 256 tile needs a quarter fewer ring
// bytes and fragment reads per MFMA.  Its accumulator is 128 registers per
// wave, so the tree fits only at one wave per SIMD and at most two saved
// levels (the current leaf and level 0 in AGPRs, level 1 in VGPRs).
//
// Layout: four waves in a 2 x 2 grid, wave tile 64 x 128 (4 x 8 blocks of
// 16 x 16).  A stage holds 64 columns of K: 128 A rows then 256 B rows of
// 128 bytes, chunks XOR-swizzled by (row & 7) as in gemm_core.hpp; three
// stages (144 KiB) form the ring.  Each k-step issues its 32 MFMAs as inline
// assembly, with one memory instruction (a fragment read for the next k-step
// or a ring load) after each of the first 18, so the matrix core keeps
// running while a memory instruction holds up the wave.  The accumulators
// are AGPR operands of those MFMAs.  The compiler does not see the MFMA
// writes, so the tree code reads a finished leaf only after explicit wait
// states (mfma_drain_w).
#pragma once

#include "gemm_core.hpp"

namespace iso {

constexpr int WBN = 256;                               // tile columns
constexpr int kWBOffset = BM * kRowBytes;              // B rows inside a stage
constexpr int kWStageBytes = (BM + WBN) * kRowBytes;   // 48 KiB
constexpr int kWBuf = 3;
constexpr int kWLdsBytes = kWBuf * kWStageBytes;       // 144 KiB

// Per-lane ring state: lane l of wave w loads A rows 32 w + 8 i + (l >> 3)
// (i < 4) and B rows 64 w + 8 i + (l >> 3) (i < 8); voff* are the byte
// offsets of those rows' swizzled 16-byte chunks.  B row groups i with bit 1
// set read through rb2 (a second source; the same as rb for one matrix).
// Rows past a matrix edge have offsets past the buffer range and read as
// zero.
struct PipeW {
    __amdgpu_buffer_rsrc_t ra, rb, rb2;
    uint32_t voffa[4];
    uint32_t voffb[8];
    uint32_t kbyte0;  // byte offset of the workgroup's first k
};
struct FragsW {
    bf16x8 a[4];
    bf16x8 b[8];
};
struct AccW {
    f32x4 v[4][8];
};

__device__ __forceinline__ PipeW make_pipe_w(const uint16_t *A_tile, int64_t rowsA,
                                             const uint16_t *B_tile, int64_t rowsB, int64_t K,
                                             int64_t k0)
{
    PipeW p;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    p.ra = tile_rsrc(A_tile, rowsA < BM ? rowsA : BM, K);
    p.rb = tile_rsrc(B_tile, rowsB < WBN ? rowsB : WBN, K);
    p.rb2 = p.rb;
    const uint32_t c = (lane & 7) ^ (lane >> 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t r = 32 * w + 8 * i + (lane >> 3);
        p.voffa[i] = (uint32_t)((int64_t)r * K * 2) + c * 16;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t r = 64 * w + 8 * i + (lane >> 3);
        p.voffb[i] = (uint32_t)((int64_t)r * K * 2) + c * 16;
    }
    p.kbyte0 = (uint32_t)(k0 * 2);
    return p;
}

// Ring load q (0..11) of stage st: q < 4 is A row group q, else B row group
// q - 4.  A stage past the end (st >= nst) reads through an empty buffer
// range (zeros into a ring slot nothing reads any more), so that every stage
// issues the same loads and the wait counts are constants.
__device__ __forceinline__ void dma_w(const PipeW &p, __amdgpu_buffer_rsrc_t rz, char *lds, int st,
                                      int nst, int q)
{
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t soff = p.kbyte0 + (uint32_t)st * (BK * 2);
    char *dst = lds + (st % kWBuf) * kWStageBytes +
                (q < 4 ? (w * 32 + q * 8) * kRowBytes
                       : kWBOffset + (w * 64 + (q - 4) * 8) * kRowBytes);
    const __amdgpu_buffer_rsrc_t r = st < nst ? (q < 4 ? p.ra : ((q - 4) & 2) ? p.rb2 : p.rb) : rz;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (ISO_LDS void *)dst, 16,
                                             q < 4 ? p.voffa[q & 3] : p.voffb[(q - 4) & 7], soff,
                                             0, 0);
}

// acc (AGPRs) += a b, or acc = a b from +0.0 for a leaf's first k-step.
// With TR the B block is the MFMA's first operand: the same products summed
// in the same order into the same element, held transposed (a lane's four
// values are four consecutive columns of one row).
template <bool FRESH, bool TR = false>
__device__ __forceinline__ void mfma_w(f32x4 &acc, const bf16x8 &a, const bf16x8 &b)
{
    if constexpr (TR) {
        if constexpr (FRESH)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&a"(acc) : "v"(b), "v"(a));
        else
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
    } else {
        if constexpr (FRESH)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&a"(acc) : "v"(a), "v"(b));
        else
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    }
}

// Fragment read R of a k-step: R < 4 is A block R, else B block R - 4.
template <int R>
__device__ __forceinline__ void frag_w(FragsW &f, uint32_t aa, uint32_t ab)
{
    if constexpr (R < 4)
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(f.a[R]) : "v"(aa), "i"(R * 16 * kRowBytes));
    else
        asm volatile("ds_read_b128 %0, %1 offset:%2"
                     : "=&v"(f.b[R - 4])
                     : "v"(ab), "i"((R - 4) * 16 * kRowBytes));
}

// One k-step: 32 MFMAs on f; after MFMA m < 18 one memory instruction, in
// the order read, read, load: the 12 fragment reads into fn (addresses aa,
// ab) and ring loads q0 .. q0+5 of stage dst.
template <bool FRESH, bool TR = false>
__device__ __forceinline__ void kstep_w(AccW &acc, const FragsW &f, FragsW &fn, uint32_t aa,
                                        uint32_t ab, const PipeW &p, __amdgpu_buffer_rsrc_t rz,
                                        char *lds, int dst, int nst, int q0)
{
    static_for<32>([&](auto Mc) {
        constexpr int m = decltype(Mc)::value;
        mfma_w<FRESH, TR>(acc.v[m / 8][m % 8], f.a[m / 8], f.b[m % 8]);
        if constexpr (m < 18) {
            if constexpr (m % 3 == 2)
                dma_w(p, rz, lds, dst, nst, q0 + m / 3);
            else
                frag_w<(m / 3) * 2 + (m % 3)>(fn, aa, ab);
        }
    });
}

// Wait for this wave's fragment reads; the registers are usable after it.
__device__ __forceinline__ void frags_wait_w(FragsW &f)
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i)
        asm volatile("" : "+v"(f.a[i]));
#pragma unroll
    for (int j = 0; j < 8; ++j)
        asm volatile("" : "+v"(f.b[j]));
}

// At most n ring loads of this wave outstanding, then a workgroup barrier
// (loads complete in order; see stage_barrier in gemm_core.hpp).
template <int N>
__device__ __forceinline__ void vm_barrier_w()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait states between the last MFMA writes of a leaf and the VALU reads of
// its sums (more than the 16x16x32 MFMA's write-to-read requirement).
__device__ __forceinline__ void mfma_drain_w(AccW &acc)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            asm volatile("" : "+a"(acc.v[i][j]));
}

// Saved sums: level 0 in AGPRs, level 1 in VGPRs (values pass unchanged).
__device__ __forceinline__ void park_w(AccW &dst, const AccW &src, bool vgpr)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            f32x4 t = src.v[i][j];
            if (vgpr)
                asm volatile("" : "=v"(t) : "0"(t));
            else
                asm volatile("" : "=a"(t) : "0"(t));
            dst.v[i][j] = t;
        }
}

// v = left + v element by element (left sibling = lower leaf indices).
__device__ __forceinline__ void unpark_add_w(AccW &v, const AccW &left)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            f32x4 t = left.v[i][j];
            f32x4 u = v.v[i][j];
            asm volatile("" : "=v"(t) : "0"(t));
            asm volatile("" : "=v"(u) : "0"(u));
            v.v[i][j] = t + u;
        }
}

template <int LOG, int J, int B>
__device__ __forceinline__ void tree_push_w(AccW (&stk)[LOG > 0 ? LOG : 1], AccW &v)
{
    if constexpr (B < LOG) {
        if constexpr (((J >> B) & 1) != 0) {
            unpark_add_w(v, stk[B]);
            tree_push_w<LOG, J, B + 1>(stk, v);
        } else {
            park_w(stk[B], v, B >= 1);
        }
    }
}

// One stage: its first k-step (fragments f0, read in the previous stage)
// reads the second k-step into f1 and issues the second half of stage st+2's
// loads; the barrier then certifies that stage st+1 landed and that every
// wave is done with stage st's fragments; the second k-step reads stage
// st+1's first k-step into f0 and issues the first half of stage st+3's
// loads into stage st's slot.  Loads of stage t are thus issued in the
// second k-step of stage t-3 and the first of stage t-2, and at the barrier
// of stage st the 12 loads of stage st+2 are the only ones issued after
// stage st+1's.
template <bool FRESH, bool TR = false>
__device__ __forceinline__ void stage_w(AccW &acc, FragsW &f0, FragsW &f1, int st, int nst,
                                        uint32_t lds_base, uint32_t rowa, uint32_t rowb,
                                        uint32_t ch0, uint32_t ch1, const PipeW &p,
                                        __amdgpu_buffer_rsrc_t rz, char *lds)
{
    const uint32_t bs = lds_base + (uint32_t)(st % kWBuf) * kWStageBytes;
    kstep_w<FRESH, TR>(acc, f0, f1, bs + rowa + ch1, bs + rowb + ch1, p, rz, lds, st + 2, nst, 6);
    frags_wait_w(f1);
    vm_barrier_w<12>();
    const uint32_t bn = lds_base + (uint32_t)((st + 1) % kWBuf) * kWStageBytes;
    kstep_w<false, TR>(acc, f1, f0, bn + rowa + ch0, bn + rowb + ch0, p, rz, lds, st + 3, nst, 0);
    frags_wait_w(f0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t empty_rsrc()
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>((const uint16_t *)nullptr),
                                             (short)0, 0, 0x00020000);
}

// The contraction of one 128 x 256 tile over 2^LOG leaves of `spl` stages
// each.  On return `root` holds the subtree root (wave (wr, wc) holds rows
// 64 wr + 16 i + 4 (lane >> 4) + r, columns 128 wc + 16 j + (lane & 15) in
// v[i][j][r]; with TR row 64 wr + 16 i + (lane & 15), columns 128 wc + 16 j
// + 4 (lane >> 4) + r), every load of this wave has landed and all waves
// have passed a final barrier, so `lds` may be reused.
template <int LOG, bool TR = false>
__device__ __forceinline__ void leaf_tree_mainloop_w(const PipeW &p, int spl, char *lds,
                                                     AccW &root)
{
    static_assert(LOG <= 2, "at most four leaves per workgroup");
    constexpr int LP = 1 << LOG;
    const int nst = LP * spl;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave >> 1, wc = wave & 1;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(ISO_LDS char *)lds;
    const uint32_t ch0 = (uint32_t)(((lane >> 4) ^ (lane & 7)) << 4);
    const uint32_t ch1 = ch0 ^ 64u;
    const uint32_t rowa = (uint32_t)(wr * 64 + (lane & 15)) * kRowBytes;
    const uint32_t rowb = (uint32_t)kWBOffset + (uint32_t)(wc * 128 + (lane & 15)) * kRowBytes;
    const __amdgpu_buffer_rsrc_t rz = empty_rsrc();

    for (int s = 0; s < 2; ++s)
        for (int q = 0; q < 12; ++q)
            dma_w(p, rz, lds, s, nst, q);
    for (int q = 0; q < 6; ++q)
        dma_w(p, rz, lds, 2, nst, q);
    vm_barrier_w<18>();  // stage 0 landed: stage 1 and half of stage 2 may be out
    FragsW f0, f1;
    static_for<12>([&](auto Rc) {
        frag_w<decltype(Rc)::value>(f0, lds_base + rowa + ch0, lds_base + rowb + ch0);
    });
    frags_wait_w(f0);
    AccW stk[LOG > 0 ? LOG : 1];
    AccW acc;
    static_for<LP>([&](auto Jc) {
        constexpr int J = decltype(Jc)::value;
        stage_w<true, TR>(acc, f0, f1, J * spl, nst, lds_base, rowa, rowb, ch0, ch1, p, rz, lds);
        for (int s = 1; s < spl; ++s)
            stage_w<false, TR>(acc, f0, f1, J * spl + s, nst, lds_base, rowa, rowb, ch0, ch1, p, rz,
                               lds);
        mfma_drain_w(acc);
        if constexpr (J < LP - 1)
            tree_push_w<LOG, J, 0>(stk, acc);
    });
    tree_push_w<LOG, LP - 1, 0>(stk, acc);
    root = acc;
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // the empty-range loads too
}

// ------------------------------------------------------------------ epilogue

// The tile's FP32 roots staged in LDS (128 rows of 1 KiB; 16-byte chunk c of
// row r at chunk c ^ (4 ((r >> 2) & 3))) so that the global stores are whole
// 16-byte vectors; the values pass unchanged.  Ends with a barrier.
__device__ __forceinline__ const float *stage_tile_w(const AccW &root, char *lds)
{
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave >> 1, wc = wave & 1;
    float *stage = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wr * 64 + i * 16 + (lane >> 4) * 4 + r;
                const int col = wc * 128 + j * 16 + (lane & 15);
                const int chunk = (col >> 2) ^ (((row >> 2) & 3) << 2);
                stage[row * WBN + chunk * 4 + (col & 3)] = root.v[i][j][r];
            }
    __syncthreads();
    return stage;
}

__device__ __forceinline__ f32x4 staged_chunk_w(const float *stage, int row, int c)
{
    return *reinterpret_cast<const f32x4 *>(stage + row * WBN +
                                            ((c ^ (((row >> 2) & 3) << 2)) << 2));
}

// Write the tile's roots to a row-major output (FP32 unchanged, or bf16
// rounded to nearest even); rows, cols: the tile's extent inside the matrix.
__device__ __forceinline__ void store_tile_w(const AccW &root, char *lds, void *out, int64_t ld,
                                             int64_t rows, int64_t cols, bool bf16_out)
{
    const float *stage = stage_tile_w(root, lds);
    const int rmax = rows < BM ? static_cast<int>(rows) : BM;
    const int cmax = cols < WBN ? static_cast<int>(cols) : WBN;
    if (bf16_out) {
        uint16_t *o = static_cast<uint16_t *>(out);
        const bool al = (reinterpret_cast<uintptr_t>(o) % 16 == 0) && (ld % 8 == 0);
        for (int u = threadIdx.x; u < BM * (WBN / 8); u += 256) {
            const int row = u / (WBN / 8), q = u % (WBN / 8);
            if (row >= rmax)
                break;
            const f32x4 lo = staged_chunk_w(stage, row, 2 * q);
            const f32x4 hi = staged_chunk_w(stage, row, 2 * q + 1);
            const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            store8_bf16(o + row * ld + 8 * q, v, al && 8 * q + 8 <= cmax, cmax - 8 * q);
        }
    } else {
        float *o = static_cast<float *>(out);
        const bool al = (reinterpret_cast<uintptr_t>(o) % 16 == 0) && (ld % 4 == 0);
        for (int u = threadIdx.x; u < BM * (WBN / 4); u += 256) {
            const int row = u / (WBN / 4), q = u % (WBN / 4);
            if (row >= rmax)
                break;
            store4_f32(o + row * ld + 4 * q, staged_chunk_w(stage, row, q),
                       al && 4 * q + 4 <= cmax, cmax - 4 * q);
        }
    }
}

}  // namespace iso
