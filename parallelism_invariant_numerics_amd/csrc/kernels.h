// kernels.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public interface is include/iso.h).  Each launcher only
// enqueues work on `stream` and returns hipGetLastError() of its launches.
// Arguments are validated by the caller (iso_host.cpp) before any launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iso {

// Leaf/tree GEMM over `parts` contiguous leaf blocks of `leaves_per_part`
// leaves (1..16) each.  mode 0: FP32 C [M][N]; 1: bf16 C; 2: FP32 partition
// roots ws[parts][M][N].
// Compute units of the current device (cached per device; 256 when the
// query fails).  Persistent kernels size their grids with it.
int device_cus();

hipError_t launch_gemm_partials(const uint16_t *A, const uint16_t *Wt, void *out, int mode,
                                int64_t M, int64_t N, int64_t K, int leaves_per_part,
                                int leaf_size, int parts, hipStream_t stream);

// The same GEMM for up to kRowsMax rows, one partition, 4-64 leaves of
// 64-512 columns, K <= kRowsMaxK (gemm_rows.hip); hipErrorNotSupported
// otherwise.  gemm_rows_supported (host code) says whether a shape
// qualifies.
constexpr int64_t kRowsMax = 256;
constexpr int64_t kRowsMaxK = 4096;
bool gemm_rows_supported(int64_t M, int64_t K, int leaves, int leaf_size);
hipError_t launch_gemm_rows(const uint16_t *A, const uint16_t *Wt, void *out, int out_bf16,
                            int64_t M, int64_t N, int64_t K, int leaves, int leaf_size,
                            hipStream_t stream);

// The same over ws[parts][M][N] written by launch_gemm_partials, tile by tile
// on the XCD that wrote each tile's roots (a grid of a multiple of 8 tiles,
// N % 4 == 0 and aligned buffers; otherwise launch_partition_combine).
hipError_t launch_partition_combine_tiles(const float *ws, void *out, int out_bf16, int64_t M,
                                          int64_t N, int parts, hipStream_t stream);

// out[e] = fixed tree over ws[0..parts)[e], e < MN; FP32 or bf16 output.
hipError_t launch_partition_combine(const float *ws, void *out, int out_bf16, int64_t MN,
                                    int parts, hipStream_t stream);

// LM-head: chunk statistics ws_stats [M][nchunk] (float2: chunk max, chunk
// exp-sum) and the target logit ws_target [M].  parts == 1 fuses the stats
// into the leaf/tree main loop; parts > 1 first writes partition roots of the
// logits to ws_roots [parts][M][V].
// Chunk statistics of the vocabulary ids [v0, v0 + V) (Wvt points at row v0
// of the vocabulary matrix; v0 a multiple of 128) of a v_total vocabulary:
// stats rows have stride ceil(v_total / 128) chunks.
hipError_t launch_lmhead_stats(const uint16_t *H, const uint16_t *Wvt, const int32_t *tok,
                               float *ws_stats, float *ws_target, float *ws_roots, int64_t M,
                               int64_t V, int64_t K, int leaves_per_part, int leaf_size,
                               int parts, int64_t v0, int64_t v_total, hipStream_t stream);

// Per row: fixed tree over the chunk statistics, then the logprob.
hipError_t launch_lmhead_finish(const float *ws_stats, const float *ws_target,
                                const int32_t *tok, float *logprob, int64_t M, int64_t V,
                                hipStream_t stream);

// RMSNorm rows: leaf_size m, chunks = elements per lane / 8 (1..16).
hipError_t launch_rmsnorm(const uint16_t *x, const uint16_t *residual, uint16_t *residual_out,
                          const uint16_t *weight, void *y, int out_bf16, int64_t M, int64_t H,
                          int leaf_size, int chunks, float eps, hipStream_t stream);

// CPR gated delta rule, head size 128, chunk C (1..64).  Prefill: chunk
// forms P, U [T/C][H][128][128], boundary states bounds [T/C + 1][H][128][128]
// (workspace), outputs o, final snap / run.  Decode: one token step of every
// head, plus the re-sync (chunk form into P, U [1][H][128][128], pass into
// snap and run) when pos closes a chunk.
hipError_t launch_cpr_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *alpha, const float *beta, const float *S0, float *o,
                              float *snap, float *run, int64_t T, int64_t H, int C, float *P,
                              float *U, float *bounds, hipStream_t stream);
hipError_t launch_cpr_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const float *alpha, const float *beta, int64_t pos, float *snap,
                             float *run, float *o, int64_t H, int C, float *P, float *U,
                             hipStream_t stream);

struct MoeBuffers {
    int32_t *idx;       // [T][k]
    float *gate;        // [T][k]
    uint16_t *h;        // [T][k][I]
    float *e;           // [T][k][H]
    int32_t *counts;    // [E]
    int32_t *rows;      // [E][T]: expert e's entries (token * k + slot) in token order, counts[e] of them
    int32_t *tiles;     // [max_tiles][4]: expert, first row within the expert, the expert's first tile, its tile count
    int32_t *ntiles;    // [1]
    int max_tiles;
    int32_t *blk_counts;  // [nblk][E] per 64-token block (two-pass bucket), or null
    int nblk;
};

// The two-pass bucket takes blocks of this many tokens, for T up to the limit.
constexpr int kMoeBucketTok = 64;
constexpr int64_t kMoeBucketMaxT = 16384;

hipError_t launch_moe(const uint16_t *X, const float *logits, const uint16_t *Wg,
                      const uint16_t *Wu, const uint16_t *Wd, float *Y, int64_t T, int64_t H,
                      int64_t E, int64_t I, int top_k, int gu_leaves, int gu_leaf_size,
                      int dn_leaves, int dn_leaf_size, const MoeBuffers &b, hipStream_t stream);

// Bytes of the LM-head's static device scratch (lmhead.hip), the workspace
// of iso_lmhead_logprob_noalloc; equals ISO_LMHEAD_NOALLOC_BYTES.
constexpr size_t kLmNoallocBytes = (size_t)32 << 20;

// Device address of that scratch on the current device, looked up with
// hipGetSymbolAddress on the first call per device and kept; the error of
// the lookup otherwise.
hipError_t lmhead_noalloc_scratch(void **ptr);

// h[i] = bf16(silu(G[i]) U[i]), act[i] (when not null) the FP32 value.
hipError_t launch_swiglu(const float *G, const float *U, float *act, uint16_t *h, int64_t n,
                         hipStream_t stream);

}  // namespace iso
