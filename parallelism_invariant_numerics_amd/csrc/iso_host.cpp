// iso_host.cpp -- the C ABI: contract validation and identity, topology
// claims, workspace sizing and kernel dispatch.  Every check runs before the
// first HIP call of an entry point.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/iso.h"
#include "kernels.h"
#include "sha256.h"

namespace {

constexpr int64_t kMaxRows = (int64_t)1 << 31;   // LM-head rows, T * top_k
constexpr int64_t kMaxDim = (int64_t)1 << 23;    // GEMM M and N (tile grid limits)
constexpr int64_t kMaxK = (int64_t)1 << 22;
constexpr int64_t kMaxVocab = (int64_t)1 << 20;  // the chunk tree's per-row fold width
constexpr int kMaxLeavesPerTile = 16;           // the kernels' register tree depth

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Contract validity for a region; chunk = the vocab_chunk the region needs.
// (the matrix-product entry points: MFMA schedule)
iso_status check_contract(const iso_contract *c, uint32_t chunk)
{
    iso_status s = iso_contract_validate(c);
    if (s != ISO_OK)
        return s;
    if (c->schedule != ISO_SCHED_MFMA16X16X32_KASC || c->vocab_chunk != chunk)
        return ISO_ERR_CONTRACT;
    return ISO_OK;
}

// Internal partition count: the caller's P, raised when a partition's leaf
// block is deeper than the register tree holds.  Raising it only moves tree
// levels from registers to the combine step; the tree is the same.
int internal_parts(const iso_contract *c, int partitions)
{
    int lpp = (int)c->leaf_count / partitions;
    return lpp > kMaxLeavesPerTile ? (int)c->leaf_count / kMaxLeavesPerTile : partitions;
}

// How an iso_gemm call runs.  The choice follows the call's shape (and
// whether a workspace was given), never the numbers, and every choice gives
// the same bits: the rows kernel, the tile kernel and the partition path
// all compute each leaf with the same MFMA chain and combine the leaves
// with the same tree.
//   rows   a few rows: one workgroup per 16 output columns streaming the
//          weights (gemm_rows.hip)
//   parts  partition roots of `parts` contiguous leaf blocks into the
//          workspace, then the top tree levels (parts == 1: the tile kernel
//          writes the output directly)
struct GemmPlan {
    bool rows;
    int parts;
};

constexpr int64_t kCus = 256;
constexpr int64_t kSmallLayerBytes = (int64_t)8 << 20;
// An internal split folds its roots tile by tile on the XCD that wrote them
// while the layer's weights leave them in that XCD's L2 (measured, same bits:
// 33-200 rows of 2048 x 2048 with 8 leaves, 2048 x 4096 with 16, 4096 x 2048
// with 4, 3072 x 2048 with 8: 10-21 % faster; on 32 MiB of weights, 4096 x
// 4096 or 8192 x 2048, 1-5 % slower, so those keep the element-order fold).
constexpr int64_t kTileFoldLayerBytes = (int64_t)16 << 20;

int64_t tile_count(int64_t M, int64_t N) { return ((M + 127) / 128) * ((N + 127) / 128); }

// P = 1 calls whose output has too few 128 x 128 tiles to fill the chip may
// split K into more partitions (whole subtrees, so the same bits) when the
// caller gives a workspace: the smallest power of two that brings the
// workgroups to one per CU, at most 8 partitions up to 64 rows and 4 above
// (the partial roots then cost more to write and fold than the extra
// workgroups gain; measured at 33-256 rows of 4096 x 4096 with 16 leaves,
// 2048 x 2048 with 8 and 4096 x 2048 with 4).
int split_parts(const iso_contract *c, int64_t M, int64_t N)
{
    const int64_t tiles = tile_count(M, N);
    int p = internal_parts(c, 1);
    if (tiles >= kCus / 2)
        return p;
    const int cap = M <= 64 ? 8 : 4;
    while (p < cap && 2 * p <= (int)c->leaf_count && tiles * p < kCus)
        p *= 2;
    return p;
}

GemmPlan plan_gemm(const iso_contract *c, int64_t M, int64_t N, int64_t K, int partitions,
                   bool have_ws)
{
    const int L = (int)c->leaf_count;
    const bool rows_ok =
        partitions == 1 && iso::gemm_rows_supported(M, K, L, (int)c->leaf_size);
    if (partitions != 1)
        return {false, internal_parts(c, partitions)};
    // weight streaming wins while the rows are few (up to 16, one MFMA row
    // block), and up to 32 rows on a layer small enough that the partition
    // roots' round trip and the second launch cost more than the rows'
    // re-reads; past that a split over the workspace, when there is one, is
    // faster (measured: 17-32 rows of 4096 x 4096 with 16 leaves 11.1-13.1 ->
    // 10.3-11.6 us, of 4096 x 2048 with 4 leaves 10.7-13.0 -> 8.9-9.6 us;
    // 48-64 rows of 2048 x 2048 with 8 leaves 9.3-10.7 -> 8.4-8.9 us)
    const bool small_layer = N * K * 2 <= kSmallLayerBytes;
    if (rows_ok && (M <= 16 || (M <= 32 && (small_layer || !have_ws))))
        return {true, 1};
    const int split = split_parts(c, M, N);
    if (split > internal_parts(c, 1) && have_ws)
        return {false, split};
    if (rows_ok && M <= 96 && L >= 8 && tile_count(M, N) < kCus / 2)
        return {true, 1};
    return {false, internal_parts(c, 1)};
}

thread_local hipError_t g_last_launch_error = hipSuccess;

iso_status launch_status(hipError_t e)
{
    g_last_launch_error = e;
    return e == hipSuccess ? ISO_OK : ISO_ERR_LAUNCH;
}

// The runtime's last-error slot may hold an error left by an earlier,
// unrelated HIP call of the caller; clear it so a launch check reports only
// this entry point's launches.
void clear_stale_error() { (void)hipGetLastError(); }

struct LmLayout {
    size_t stats, target, roots, total;
};

LmLayout lm_layout(int64_t M, int64_t V, int parts)
{
    const int64_t nchunk = (V + ISO_VOCAB_CHUNK - 1) / ISO_VOCAB_CHUNK;
    LmLayout l;
    l.stats = 0;
    l.target = align_up((size_t)M * (size_t)nchunk * 2 * sizeof(float));
    l.roots = l.target + align_up((size_t)M * sizeof(float));
    l.total = l.roots + (parts > 1 ? align_up((size_t)parts * M * V * sizeof(float)) : 0);
    return l;
}

iso_status check_gemm_shape(const iso_contract *c, int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0)
        return ISO_ERR_ARG;
    if (K != (int64_t)c->leaf_count * c->leaf_size)
        return ISO_ERR_SHAPE;
    if (M >= kMaxRows || N >= kMaxRows || K > kMaxK)
        return ISO_ERR_SHAPE;
    return ISO_OK;
}

// The tile grid is one-dimensional: (M/128) * (N/128) * 8 partitions must
// stay below 2^31 workgroups.
iso_status check_gemm_dims(int64_t M, int64_t N)
{
    if (M >= kMaxDim || N >= kMaxDim)
        return ISO_ERR_SHAPE;
    return ((M + 127) / 128) * ((N + 127) / 128) * 8 < ((int64_t)1 << 31) ? ISO_OK
                                                                          : ISO_ERR_SHAPE;
}

}  // namespace

namespace iso {

// The shapes the weight-streaming kernel takes: whole 32-column k-steps,
// four leaves (two column blocks of four subtrees) or 8-64 leaves (eight
// subtrees), at most 16 k-steps per wave.
bool gemm_rows_supported(int64_t M, int64_t K, int leaves, int leaf_size)
{
    if (M < 1 || M > kRowsMax || K > kRowsMaxK || leaf_size % 32 != 0)
        return false;
    const int ks = leaf_size / 32;
    if (static_cast<int64_t>(ks) * 32 * leaves != K)
        return false;
    if (leaves != 4 && leaves != 8 && leaves != 16 && leaves != 32 && leaves != 64)
        return false;
    const int lw = leaves == 4 ? 1 : leaves / 8;  // leaves per wave
    return (ks == 2 || ks == 4 || ks == 8 || ks == 16) && lw * ks <= 16;
}

}  // namespace iso

extern "C" {

iso_status iso_contract_init(iso_contract *c, uint32_t leaf_count, uint32_t leaf_size,
                             uint32_t vocab_chunk)
{
    if (!c)
        return ISO_ERR_ARG;
    c->abi_version = ISO_ABI_VERSION;
    c->in_dtype = ISO_BF16;
    c->accum_dtype = ISO_F32;
    c->leaf_count = leaf_count;
    c->leaf_size = leaf_size;
    c->tree = ISO_TREE_BALANCED;
    c->vocab_chunk = vocab_chunk;
    c->schedule = ISO_SCHED_MFMA16X16X32_KASC;
    return ISO_OK;
}

iso_status iso_contract_validate(const iso_contract *c)
{
    if (!c)
        return ISO_ERR_ARG;
    if (c->abi_version != ISO_ABI_VERSION)
        return ISO_ERR_CONTRACT;
    if (c->in_dtype != ISO_BF16 || c->accum_dtype != ISO_F32)
        return ISO_ERR_DTYPE;
    if (c->tree != ISO_TREE_BALANCED)
        return ISO_ERR_CONTRACT;
    if (c->schedule == ISO_SCHED_MFMA16X16X32_KASC) {
        if (!is_pow2(c->leaf_count) || c->leaf_count > 64)
            return ISO_ERR_CONTRACT;
        if (c->leaf_size < 64 || c->leaf_size > 65536 || c->leaf_size % 64 != 0)
            return ISO_ERR_CONTRACT;
        if (c->vocab_chunk != 0 && c->vocab_chunk != ISO_VOCAB_CHUNK)
            return ISO_ERR_CONTRACT;
        return ISO_OK;
    }
    if (c->schedule == ISO_SCHED_SEQ_KASC) {
        if (!is_pow2(c->leaf_count) || c->leaf_count > 4096)
            return ISO_ERR_CONTRACT;
        if (c->leaf_size < 1 || c->leaf_size > 65536 || c->vocab_chunk != 0)
            return ISO_ERR_CONTRACT;
        return ISO_OK;
    }
    if (c->schedule == ISO_SCHED_CPR_GDN) {
        if (!is_pow2(c->leaf_count) || c->leaf_count > 4096)
            return ISO_ERR_CONTRACT;
        if (c->leaf_size < 1 || c->leaf_size > 64 || c->vocab_chunk != 0)
            return ISO_ERR_CONTRACT;
        return ISO_OK;
    }
    return ISO_ERR_CONTRACT;
}

iso_status iso_contract_digest(const iso_contract *c, uint8_t out[32])
{
    if (!out)
        return ISO_ERR_ARG;
    iso_status s = iso_contract_validate(c);
    if (s != ISO_OK)
        return s;
    static const char kTag[] = "iso.numerical_policy.v1";  // 23 chars + NUL
    static_assert(sizeof(kTag) == 24, "tag is 24 bytes with its NUL");
    uint8_t msg[24 + 32];
    memcpy(msg, kTag, 24);
    const uint32_t f[8] = {c->abi_version, c->in_dtype, c->accum_dtype, c->leaf_count,
                           c->leaf_size, c->tree, c->vocab_chunk, c->schedule};
    for (int i = 0; i < 8; ++i)
        for (int b = 0; b < 4; ++b)
            msg[24 + 4 * i + b] = (uint8_t)(f[i] >> (8 * b));
    iso::sha256(msg, sizeof msg, out);
    return ISO_OK;
}

iso_status iso_contract_check(const iso_contract *c, const uint8_t want[32])
{
    if (!want)
        return ISO_ERR_ARG;
    uint8_t got[32];
    iso_status s = iso_contract_digest(c, got);
    if (s != ISO_OK)
        return s;
    return memcmp(got, want, 32) == 0 ? ISO_OK : ISO_ERR_IDENTITY;
}

iso_status iso_check_partitions(const iso_contract *c, int partitions)
{
    iso_status s = iso_contract_validate(c);
    if (s != ISO_OK)
        return s;
    if (partitions != 1 && partitions != 2 && partitions != 4 && partitions != 8)
        return ISO_ERR_CLAIM;
    if ((int)c->leaf_count % partitions != 0)
        return ISO_ERR_CLAIM;
    return ISO_OK;
}

size_t iso_gemm_workspace(const iso_contract *c, int64_t M, int64_t N, int partitions)
{
    if (check_contract(c, 0) != ISO_OK || iso_check_partitions(c, partitions) != ISO_OK)
        return (size_t)-1;
    if (M < 0 || N < 0 || M >= kMaxDim || N >= kMaxDim)
        return (size_t)-1;
    const int64_t K = (int64_t)c->leaf_count * c->leaf_size;
    const int parts = plan_gemm(c, M, N, K, partitions, true).parts;
    return parts > 1 ? (size_t)parts * (size_t)M * (size_t)N * sizeof(float) : 0;
}

iso_status iso_gemm(const iso_contract *c, const void *A, const void *Wt, void *C,
                    uint32_t out_dtype, int64_t M, int64_t N, int64_t K, int partitions,
                    void *workspace, size_t workspace_bytes, void *stream)
{
    iso_status s = check_contract(c, 0);
    if (s != ISO_OK)
        return s;
    if ((s = check_gemm_shape(c, M, N, K)) != ISO_OK)
        return s;
    if ((s = check_gemm_dims(M, N)) != ISO_OK)
        return s;
    if (out_dtype != ISO_F32 && out_dtype != ISO_BF16)
        return ISO_ERR_DTYPE;
    if ((s = iso_check_partitions(c, partitions)) != ISO_OK)
        return s;
    if (M == 0 || N == 0)
        return ISO_OK;
    if (!A || !Wt || !C || !aligned16(A) || !aligned16(Wt))
        return ISO_ERR_ARG;
    // a P = 1 call may take the split-K plan only with a workspace big
    // enough for it; without one it runs another plan with the same bits
    const size_t split_need = iso_gemm_workspace(c, M, N, partitions);
    const bool have_ws = workspace && workspace_bytes >= split_need;
    const GemmPlan plan = plan_gemm(c, M, N, K, partitions, have_ws);
    const int parts = plan.parts;
    const size_t need = parts > 1 ? (size_t)parts * (size_t)M * (size_t)N * sizeof(float) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need))
        return ISO_ERR_WORKSPACE;

    clear_stale_error();
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int lpp = (int)c->leaf_count / parts;
    const int bf16 = out_dtype == ISO_BF16;
    if (plan.rows)
        return launch_status(iso::launch_gemm_rows(
            static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(Wt), C, bf16, M, N, K,
            (int)c->leaf_count, (int)c->leaf_size, st));
    if (parts == 1)
        return launch_status(iso::launch_gemm_partials(
            static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(Wt), C, bf16 ? 1 : 0,
            M, N, K, lpp, (int)c->leaf_size, 1, st));
    hipError_t e = iso::launch_gemm_partials(static_cast<const uint16_t *>(A),
                                             static_cast<const uint16_t *>(Wt), workspace, 2, M,
                                             N, K, lpp, (int)c->leaf_size, parts, st);
    if (e != hipSuccess)
        return launch_status(e);
    if (partitions == 1 && N * K * 2 <= kTileFoldLayerBytes)
        return launch_status(iso::launch_partition_combine_tiles(
            static_cast<const float *>(workspace), C, bf16, M, N, parts, st));
    return launch_status(iso::launch_partition_combine(static_cast<const float *>(workspace), C,
                                                       bf16, M * N, parts, st));
}

iso_status iso_gemm_baseline(const void *A, const void *Wt, void *C, uint32_t out_dtype,
                             int64_t M, int64_t N, int64_t K, void *stream)
{
    if (M < 0 || N < 0 || K < 0)
        return ISO_ERR_ARG;
    if (K == 0 || K % 64 != 0 || K > kMaxK || M >= kMaxDim || N >= kMaxDim)
        return ISO_ERR_SHAPE;
    if (out_dtype != ISO_F32 && out_dtype != ISO_BF16)
        return ISO_ERR_DTYPE;
    if (M == 0 || N == 0)
        return ISO_OK;
    if (!A || !Wt || !C || !aligned16(A) || !aligned16(Wt))
        return ISO_ERR_ARG;
    // one leaf spanning all of K: a single accumulator, no tree
    clear_stale_error();
    return launch_status(iso::launch_gemm_partials(
        static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(Wt), C,
        out_dtype == ISO_BF16 ? 1 : 0, M, N, K, 1, (int)K, 1, static_cast<hipStream_t>(stream)));
}

size_t iso_lmhead_workspace(const iso_contract *c, int64_t M, int64_t V, int partitions)
{
    if (check_contract(c, ISO_VOCAB_CHUNK) != ISO_OK ||
        iso_check_partitions(c, partitions) != ISO_OK)
        return (size_t)-1;
    if (M < 0 || V < 1 || M >= kMaxRows || V > kMaxVocab)
        return (size_t)-1;
    return lm_layout(M, V, internal_parts(c, partitions)).total;
}

iso_status iso_lmhead_logprob(const iso_contract *c, const void *H, const void *Wvt,
                              const int32_t *tok, float *logprob, int64_t M, int64_t V,
                              int64_t K, int partitions, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    iso_status s = check_contract(c, ISO_VOCAB_CHUNK);
    if (s != ISO_OK)
        return s;
    if ((s = check_gemm_shape(c, M, V, K)) != ISO_OK)
        return s;
    if (V < 1 || V > kMaxVocab)
        return ISO_ERR_SHAPE;
    if (((M + 127) / 128) * ((V + 127) / 128) >= ((int64_t)1 << 31))
        return ISO_ERR_SHAPE;
    if ((s = iso_check_partitions(c, partitions)) != ISO_OK)
        return s;
    if (M == 0)
        return ISO_OK;
    if (!H || !Wvt || !tok || !logprob || !aligned16(H) || !aligned16(Wvt))
        return ISO_ERR_ARG;
    const int parts = internal_parts(c, partitions);
    const LmLayout l = lm_layout(M, V, parts);
    if (!workspace || workspace_bytes < l.total || !aligned16(workspace))
        return ISO_ERR_WORKSPACE;

    clear_stale_error();
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    float *stats = reinterpret_cast<float *>(ws + l.stats);
    float *target = reinterpret_cast<float *>(ws + l.target);
    float *roots = parts > 1 ? reinterpret_cast<float *>(ws + l.roots) : nullptr;
    hipError_t e = iso::launch_lmhead_stats(
        static_cast<const uint16_t *>(H), static_cast<const uint16_t *>(Wvt), tok, stats, target,
        roots, M, V, K, (int)c->leaf_count / parts, (int)c->leaf_size, parts, 0, V, st);
    if (e != hipSuccess)
        return launch_status(e);
    return launch_status(iso::launch_lmhead_finish(stats, target, tok, logprob, M, V, st));
}

iso_status iso_lmhead_logprob_noalloc(const iso_contract *c, const void *H, const void *Wvt,
                                      const int32_t *tok, float *logprob, int64_t M, int64_t V,
                                      int64_t K, void *stream)
{
    static_assert(iso::kLmNoallocBytes == ISO_LMHEAD_NOALLOC_BYTES, "one scratch size");
    iso_status s = check_contract(c, ISO_VOCAB_CHUNK);
    if (s != ISO_OK)
        return s;
    if ((s = check_gemm_shape(c, M, V, K)) != ISO_OK)
        return s;
    if (V < 1 || V > kMaxVocab)
        return ISO_ERR_SHAPE;
    if (M == 0)
        return ISO_OK;
    if (!H || !Wvt || !tok || !logprob || !aligned16(H) || !aligned16(Wvt))
        return ISO_ERR_ARG;
    const int parts = internal_parts(c, 1);
    const LmLayout l = lm_layout(M, V, parts);
    if (l.total > ISO_LMHEAD_NOALLOC_BYTES)
        return ISO_ERR_WORKSPACE;

    clear_stale_error();
    void *scratch = nullptr;
    const hipError_t se = iso::lmhead_noalloc_scratch(&scratch);
    if (se != hipSuccess)
        return launch_status(se);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(scratch);
    float *stats = reinterpret_cast<float *>(ws + l.stats);
    float *target = reinterpret_cast<float *>(ws + l.target);
    float *roots = parts > 1 ? reinterpret_cast<float *>(ws + l.roots) : nullptr;
    hipError_t e = iso::launch_lmhead_stats(
        static_cast<const uint16_t *>(H), static_cast<const uint16_t *>(Wvt), tok, stats, target,
        roots, M, V, K, (int)c->leaf_count / parts, (int)c->leaf_size, parts, 0, V, st);
    if (e != hipSuccess)
        return launch_status(e);
    return launch_status(iso::launch_lmhead_finish(stats, target, tok, logprob, M, V, st));
}

iso_status iso_lmhead_shard_stats(const iso_contract *c, const void *H, const void *Wvt_shard,
                                  const int32_t *tok, float *stats, float *target, int64_t M,
                                  int64_t V, int64_t v_begin, int64_t v_end, int64_t K,
                                  void *stream)
{
    iso_status s = check_contract(c, ISO_VOCAB_CHUNK);
    if (s != ISO_OK)
        return s;
    if (V < 1 || V > kMaxVocab)
        return ISO_ERR_SHAPE;
    if (v_begin < 0 || v_end <= v_begin || v_end > V || v_begin % ISO_VOCAB_CHUNK != 0 ||
        (v_end != V && v_end % ISO_VOCAB_CHUNK != 0))
        return ISO_ERR_SHAPE;  // whole chunks, the last one may be ragged at V
    const int64_t Vs = v_end - v_begin;
    if ((s = check_gemm_shape(c, M, Vs, K)) != ISO_OK)
        return s;
    if (((M + 127) / 128) * ((Vs + 127) / 128) >= ((int64_t)1 << 31))
        return ISO_ERR_SHAPE;
    if ((int)c->leaf_count > kMaxLeavesPerTile)
        return ISO_ERR_CLAIM;  // one partition: the register tree holds at most 16 leaves
    if (M == 0)
        return ISO_OK;
    if (!H || !Wvt_shard || !tok || !stats || !target || !aligned16(H) || !aligned16(Wvt_shard))
        return ISO_ERR_ARG;
    clear_stale_error();
    return launch_status(iso::launch_lmhead_stats(
        static_cast<const uint16_t *>(H), static_cast<const uint16_t *>(Wvt_shard), tok, stats,
        target, nullptr, M, Vs, K, (int)c->leaf_count, (int)c->leaf_size, 1, v_begin, V,
        static_cast<hipStream_t>(stream)));
}
iso_status iso_lmhead_finish(const float *stats, const float *target, const int32_t *tok,
                             float *logprob, int64_t M, int64_t V, void *stream)
{
    if (M < 0 || V < 1)
        return ISO_ERR_ARG;
    if (V > kMaxVocab || M >= kMaxRows)
        return ISO_ERR_SHAPE;
    if (M == 0)
        return ISO_OK;
    if (!stats || !target || !tok || !logprob)
        return ISO_ERR_ARG;
    clear_stale_error();
    return launch_status(
        iso::launch_lmhead_finish(stats, target, tok, logprob, M, V, static_cast<hipStream_t>(stream)));
}
namespace {

struct MoeFull {
    iso_moe_layout pub;
    size_t counts, rows, tiles, ntiles, blk;
    int max_tiles;
    int nblk;  // 64-token blocks of the two-pass bucket (0: one pass per expert)
};

iso_status moe_dims(int64_t T, int64_t H, int64_t E, int64_t I, int top_k)
{
    if (T < 0 || H < 1 || I < 1 || E < 1 || top_k < 1)
        return ISO_ERR_ARG;
    if (E > 1024 || top_k > 16 || top_k > E)
        return ISO_ERR_SHAPE;
    if (H % 64 != 0 || I % 64 != 0 || H > kMaxK || I > kMaxK)
        return ISO_ERR_SHAPE;
    if (T * top_k >= kMaxRows || T * H * 2 >= ((int64_t)1 << 32) ||
        T * top_k * I * 2 >= ((int64_t)1 << 32) || I * H * 2 >= ((int64_t)1 << 32))
        return ISO_ERR_SHAPE;
    return ISO_OK;
}

MoeFull moe_layout(int64_t T, int64_t H, int64_t E, int64_t I, int top_k)
{
    MoeFull l;
    const size_t tk = (size_t)T * top_k;
    size_t o = 0;
    l.pub.idx = o;
    o += align_up(tk * 4);
    l.pub.gate = o;
    o += align_up(tk * 4);
    l.pub.h = o;
    o += align_up(tk * (size_t)I * 2);
    l.pub.e = o;
    o += align_up(tk * (size_t)H * 4);
    l.counts = o;
    o += align_up((size_t)E * 4);
    l.rows = o;
    o += align_up((size_t)E * (size_t)T * 4);
    l.max_tiles = (int)(E + (tk + 127) / 128);
    l.tiles = o;
    o += align_up((size_t)l.max_tiles * 4 * 4);
    l.ntiles = o;
    o += 256;
    // per-block expert counts of the two-pass bucket (at most 16384 tokens)
    l.nblk = T <= iso::kMoeBucketMaxT ? (int)((T + iso::kMoeBucketTok - 1) / iso::kMoeBucketTok) : 0;
    l.blk = o;
    o += align_up((size_t)l.nblk * (size_t)E * 4);
    l.pub.total = o;
    return l;
}

}  // namespace

iso_status iso_rmsnorm(const iso_contract *c, const void *x, const void *residual,
                       void *residual_out, const void *weight, void *y, uint32_t out_dtype,
                       int64_t M, int64_t H, float eps, void *stream)
{
    iso_status s = iso_contract_validate(c);
    if (s != ISO_OK)
        return s;
    if (c->schedule != ISO_SCHED_SEQ_KASC)
        return ISO_ERR_CONTRACT;
    if (M < 0 || H < 1)
        return ISO_ERR_ARG;
    if (H != (int64_t)c->leaf_count * c->leaf_size || H % 8 != 0 || M >= kMaxRows)
        return ISO_ERR_SHAPE;
    // one wave per row: each lane holds one leaf, or L/64 whole leaves
    const int64_t lanes = c->leaf_count < 64 ? (int64_t)c->leaf_count : 64;
    const int64_t span = H / lanes;  // elements per lane
    if (span < 8 || span > 128 || !is_pow2(span))
        return ISO_ERR_SHAPE;
    if (span % c->leaf_size != 0 || span / c->leaf_size > 8)
        return ISO_ERR_SHAPE;
    if (out_dtype != ISO_F32 && out_dtype != ISO_BF16)
        return ISO_ERR_DTYPE;
    if (!(eps >= 0.0f) || eps > 3.0e38f)
        return ISO_ERR_ARG;
    if (M == 0)
        return ISO_OK;
    if (!x || !weight || !y || !aligned16(x) || !aligned16(weight) || !aligned16(y))
        return ISO_ERR_ARG;
    if (y == x || y == residual || y == residual_out || residual_out == x)
        return ISO_ERR_ARG;
    if ((residual && !aligned16(residual)) || (residual_out && !aligned16(residual_out)))
        return ISO_ERR_ARG;
    clear_stale_error();
    return launch_status(iso::launch_rmsnorm(
        static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(residual),
        static_cast<uint16_t *>(residual_out), static_cast<const uint16_t *>(weight), y,
        out_dtype == ISO_BF16 ? 1 : 0, M, H, (int)c->leaf_size, (int)(span / 8), eps,
        static_cast<hipStream_t>(stream)));
}
namespace {

constexpr int64_t kCprHead = 128;

struct CprLayout {
    size_t P, U, bounds, total;
};

CprLayout cpr_layout(int64_t H, int64_t T, int64_t C)
{
    const size_t state = (size_t)H * kCprHead * kCprHead * sizeof(float);
    const size_t nb = (size_t)(T / C);
    CprLayout l;
    l.P = 0;
    l.U = align_up(nb * state);
    l.bounds = l.U + align_up(nb * state);
    l.total = l.bounds + align_up((nb + 1) * state);
    return l;
}

iso_status cpr_check(const iso_contract *c, int64_t H, int64_t T)
{
    iso_status s = iso_contract_validate(c);
    if (s != ISO_OK)
        return s;
    if (c->schedule != ISO_SCHED_CPR_GDN)
        return ISO_ERR_CONTRACT;
    if (c->leaf_count != kCprHead)
        return ISO_ERR_SHAPE;
    if (H < 1 || H >= 65536 || T < 0)
        return ISO_ERR_ARG;
    if ((T + c->leaf_size - 1) / c->leaf_size >= 65536)
        return ISO_ERR_SHAPE;
    return ISO_OK;
}

}  // namespace

size_t iso_cpr_workspace(const iso_contract *c, int64_t H, int64_t T)
{
    if (cpr_check(c, H, T) != ISO_OK)
        return (size_t)-1;
    return cpr_layout(H, T, c->leaf_size).total;
}

iso_status iso_cpr_prefill(const iso_contract *c, const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta, const float *S0, float *o,
                           float *snap, float *run, int64_t T, int64_t H, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    iso_status s = cpr_check(c, H, T);
    if (s != ISO_OK)
        return s;
    if (!snap || !run || snap == run || !aligned16(snap) || !aligned16(run))
        return ISO_ERR_ARG;
    if (S0 && !aligned16(S0))
        return ISO_ERR_ARG;
    if (T > 0) {
        if (!q || !k || !v || !alpha || !beta || !o)
            return ISO_ERR_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
            return ISO_ERR_ARG;
        const void *ins[] = {q, k, v, alpha, beta, S0, snap, run};
        for (const void *p : ins)
            if (p == (const void *)o)
                return ISO_ERR_ARG;
    }
    const CprLayout l = cpr_layout(H, T, c->leaf_size);
    if (!workspace || workspace_bytes < l.total || !aligned16(workspace))
        return ISO_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    clear_stale_error();
    return launch_status(iso::launch_cpr_prefill(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), alpha, beta, S0, o, snap, run, T, H, (int)c->leaf_size,
        reinterpret_cast<float *>(ws + l.P), reinterpret_cast<float *>(ws + l.U),
        reinterpret_cast<float *>(ws + l.bounds), static_cast<hipStream_t>(stream)));
}

iso_status iso_cpr_decode_step(const iso_contract *c, const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta, int64_t pos, float *snap,
                               float *run, float *o, int64_t H, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    iso_status s = cpr_check(c, H, c ? (int64_t)c->leaf_size : 0);
    if (s != ISO_OK)
        return s;
    if (pos < 0 || pos >= ((int64_t)1 << 40))
        return ISO_ERR_ARG;
    if (!q || !k || !v || !alpha || !beta || !o || !snap || !run || snap == run)
        return ISO_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(snap) ||
        !aligned16(run))
        return ISO_ERR_ARG;
    const void *ins[] = {q, k, v, alpha, beta, snap, run};
    for (const void *p : ins)
        if (p == (const void *)o)
            return ISO_ERR_ARG;
    const CprLayout l = cpr_layout(H, c->leaf_size, c->leaf_size);
    if (!workspace || workspace_bytes < l.total || !aligned16(workspace))
        return ISO_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    clear_stale_error();
    return launch_status(iso::launch_cpr_decode(
        static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
        static_cast<const uint16_t *>(v), alpha, beta, pos, snap, run, o, H, (int)c->leaf_size,
        reinterpret_cast<float *>(ws + l.P), reinterpret_cast<float *>(ws + l.U),
        static_cast<hipStream_t>(stream)));
}

iso_status iso_moe_layout_of(int64_t T, int64_t H, int64_t E, int64_t I, int top_k,
                             iso_moe_layout *out)
{
    if (!out)
        return ISO_ERR_ARG;
    iso_status s = moe_dims(T, H, E, I, top_k);
    if (s != ISO_OK)
        return s;
    *out = moe_layout(T, H, E, I, top_k).pub;
    return ISO_OK;
}

size_t iso_moe_workspace(int64_t T, int64_t H, int64_t E, int64_t I, int top_k)
{
    if (moe_dims(T, H, E, I, top_k) != ISO_OK)
        return (size_t)-1;
    return moe_layout(T, H, E, I, top_k).pub.total;
}

iso_status iso_moe_combine(const iso_contract *gate_up, const iso_contract *down,
                           const void *X, const float *router_logits, const void *Wg,
                           const void *Wu, const void *Wd, float *Y, int64_t T, int64_t H,
                           int64_t E, int64_t I, int top_k, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    iso_status s = check_contract(gate_up, 0);
    if (s != ISO_OK)
        return s;
    if ((s = check_contract(down, 0)) != ISO_OK)
        return s;
    if ((s = moe_dims(T, H, E, I, top_k)) != ISO_OK)
        return s;
    if (H != (int64_t)gate_up->leaf_count * gate_up->leaf_size ||
        I != (int64_t)down->leaf_count * down->leaf_size)
        return ISO_ERR_SHAPE;
    if (gate_up->leaf_count > (uint32_t)kMaxLeavesPerTile ||
        down->leaf_count > (uint32_t)kMaxLeavesPerTile)
        return ISO_ERR_SHAPE;
    if (T == 0)
        return ISO_OK;
    if (!X || !router_logits || !Wg || !Wu || !Wd || !Y || !aligned16(X) || !aligned16(Wg) ||
        !aligned16(Wu) || !aligned16(Wd) || !aligned16(Y))
        return ISO_ERR_ARG;
    const MoeFull l = moe_layout(T, H, E, I, top_k);
    if (!workspace || workspace_bytes < l.pub.total || ((uintptr_t)workspace & 255u) != 0)
        return ISO_ERR_WORKSPACE;

    clear_stale_error();
    char *ws = static_cast<char *>(workspace);
    iso::MoeBuffers b;
    b.idx = reinterpret_cast<int32_t *>(ws + l.pub.idx);
    b.gate = reinterpret_cast<float *>(ws + l.pub.gate);
    b.h = reinterpret_cast<uint16_t *>(ws + l.pub.h);
    b.e = reinterpret_cast<float *>(ws + l.pub.e);
    b.counts = reinterpret_cast<int32_t *>(ws + l.counts);
    b.rows = reinterpret_cast<int32_t *>(ws + l.rows);
    b.tiles = reinterpret_cast<int32_t *>(ws + l.tiles);
    b.ntiles = reinterpret_cast<int32_t *>(ws + l.ntiles);
    b.max_tiles = l.max_tiles;
    b.blk_counts = l.nblk > 0 ? reinterpret_cast<int32_t *>(ws + l.blk) : nullptr;
    b.nblk = l.nblk;
    return launch_status(iso::launch_moe(
        static_cast<const uint16_t *>(X), router_logits, static_cast<const uint16_t *>(Wg),
        static_cast<const uint16_t *>(Wu), static_cast<const uint16_t *>(Wd), Y, T, H, E, I,
        top_k, (int)gate_up->leaf_count, (int)gate_up->leaf_size, (int)down->leaf_count,
        (int)down->leaf_size, b, static_cast<hipStream_t>(stream)));
}

iso_status iso_swiglu(const float *G, const float *U, float *act, void *h, int64_t n,
                      void *stream)
{
    if (n < 0)
        return ISO_ERR_ARG;
    if (n == 0)
        return ISO_OK;
    if (!G || !U || !h)
        return ISO_ERR_ARG;
    clear_stale_error();
    return launch_status(iso::launch_swiglu(G, U, act, static_cast<uint16_t *>(h), n,
                                            static_cast<hipStream_t>(stream)));
}

const char *iso_status_str(iso_status s)
{
    switch (s) {
    case ISO_OK: return "ok";
    case ISO_ERR_ARG: return "invalid argument";
    case ISO_ERR_SHAPE: return "shape does not fit the contract or the size limits";
    case ISO_ERR_DTYPE: return "unsupported dtype";
    case ISO_ERR_CLAIM: return "partition count outside the contract's topology claim";
    case ISO_ERR_IDENTITY: return "contract digest differs from the expected identity";
    case ISO_ERR_WORKSPACE: return "workspace missing or too small";
    case ISO_ERR_LAUNCH: return "kernel launch failed";
    case ISO_ERR_CONTRACT: return "malformed contract";
    }
    return "unknown status";
}

const char *iso_version(void) { return "iso 0.1.0 gfx950"; }

const char *iso_last_launch_error(void) { return hipGetErrorString(g_last_launch_error); }

}  // extern "C"
