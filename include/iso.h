/*
 * iso.h -- C ABI of the parallelism- and batch-invariant matmul and
 * token-logprob library for AMD MI355X (gfx950).
 *
 * Pages cited (web pages about IsoExec):
 *   [AGL] "IsoExec: Eliminating Trainer-Inference Mismatch in SkyRL"
 *         (agentlenshq.com blog summary)
 *   [KTB] katelyatop-blog.pages.dev post on vLLM/SkyRL IsoExec and the
 *         trainer-inference mismatch (numbered sections)
 *   [DDV] "IsoExec: Unified Execution to Eliminate Trainer-Inference
 *         Mismatch in SkyRL" (daily.dev summary)
 *
 * Numerics common to every entry point.  A contraction over K is cut into
 * `leaf_count` contiguous leaves of `leaf_size`; each leaf is a bf16 dot
 * product accumulated in FP32 with one fixed MFMA schedule; the leaf sums are
 * combined by the balanced binary tree in leaf-index order (pairs (2i, 2i+1)
 * at every level) ([AGL] "Achieving Parallelism Invariance", TP bullet;
 * [KTB] section 8).  The bits of an output element therefore depend only on
 * its own input row, its own weight column and the contract -- not on the
 * batch size, the row's position in the batch, the tiling, or the number of
 * partitions ("emulated ranks") the leaves are spread over ([AGL] "Contract
 * Structure and Enforcement": composition pins the reduction decomposition,
 * claims list the parallel sizes for which the tree is proven invariant).
 *
 * Conventions.
 *   - Memory: every tensor pointer is a DEVICE pointer owned by the caller,
 *     row-major and contiguous.  bf16 tensors are raw 16-bit patterns.
 *     Weights are stored k-contiguous: a K x N matrix W is passed as its
 *     transpose Wt [N][K] (the storage of a linear layer's weight).
 *   - Workspace: the caller passes device scratch of at least the size the
 *     matching *_workspace() function returns (may be 0 / NULL when that
 *     size is 0).  The library allocates and frees nothing.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  Work is
 *     only enqueued; nothing synchronises.  No global mutable state: calls are
 *     thread-safe; calls that share a workspace must be ordered by the caller.
 *   - Errors: every argument, shape, dtype, claim and workspace check runs on
 *     the host before anything is launched; on error nothing is written and
 *     no HIP call is made.  ISO_ERR_LAUNCH reports a failed launch; device
 *     faults surface at the caller's next synchronisation.
 *   - Sizes are int64_t; M, N, K, V, T >= 0; an empty problem (M == 0 or
 *     N == 0) returns ISO_OK without launching.
 */
#ifndef ISO_H_
#define ISO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ISO_ABI_VERSION 1u

typedef enum iso_status {
    ISO_OK = 0,
    ISO_ERR_ARG = 1,        /* null pointer, bad enum value, negative size */
    ISO_ERR_SHAPE = 2,      /* K != leaf_count * leaf_size, size limits exceeded */
    ISO_ERR_DTYPE = 3,      /* unsupported input / accumulation / output dtype */
    ISO_ERR_CLAIM = 4,      /* partition count outside the contract's claims */
    ISO_ERR_IDENTITY = 5,   /* contract digest differs from the expected one */
    ISO_ERR_WORKSPACE = 6,  /* workspace missing or too small */
    ISO_ERR_LAUNCH = 7,     /* a kernel launch failed */
    ISO_ERR_CONTRACT = 8    /* malformed contract (version, leaf shape, tree, schedule) */
} iso_status;

/* dtypes */
#define ISO_BF16 1u
#define ISO_F32 2u

/* tree: the balanced binary tree over leaf index, lower index on the left */
#define ISO_TREE_BALANCED 1u
/* schedule: bf16 MFMA 16x16x32 (v_mfma_f32_16x16x32_bf16), FP32 accumulator,
 * K ascending in steps of 32 inside each leaf; the leaf sum starts at +0.0 */
#define ISO_SCHED_MFMA16X16X32_KASC 1u
/* schedule: FP32 sum of the leaf's terms one at a time in ascending index
 * order, starting at +0.0 (reductions that are not matrix products) */
#define ISO_SCHED_SEQ_KASC 2u
/* schedule: CPR gated delta rule (iso_cpr_prefill, iso_cpr_decode_step):
 * leaf_count = head size d (the dot products are balanced trees over d
 * single-product leaves), leaf_size = chunk length C (the state re-sync
 * interval), every operation a single FP32 multiply or add */
#define ISO_SCHED_CPR_GDN 3u

/* Vocabulary chunk width of the LM-head softmax (its leaf size). */
#define ISO_VOCAB_CHUNK 128u

/*
 * The numerical-policy part of an execution contract, one per region (one
 * kernel-implemented arithmetic span: gemm, lmhead, moe gate/up, moe down)
 * ([AGL] "Contract Structure and Enforcement": regions, composition with
 * pinned accumulation dtype and reduction-decomposition parameters).
 *   abi_version  ISO_ABI_VERSION
 *   in_dtype     ISO_BF16 (only)
 *   accum_dtype  ISO_F32 (only)
 *   leaf_count   L: power of two, 1..64 (MFMA schedule), 1..4096 (sequential)
 *   leaf_size    m: multiple of 64, 64..65536 (MFMA schedule), 1..65536
 *                (sequential); the reduced length (K, H) must equal L * m
 *   tree         ISO_TREE_BALANCED (only)
 *   vocab_chunk  ISO_VOCAB_CHUNK for iso_lmhead_logprob, 0 otherwise
 *   schedule     ISO_SCHED_MFMA16X16X32_KASC for iso_gemm, iso_lmhead_logprob
 *                and iso_moe_combine; ISO_SCHED_SEQ_KASC for iso_rmsnorm;
 *                ISO_SCHED_CPR_GDN for the CPR entry points (leaf_count = d,
 *                a power of two up to 4096; leaf_size = C, 1..64)
 */
typedef struct iso_contract {
    uint32_t abi_version;
    uint32_t in_dtype;
    uint32_t accum_dtype;
    uint32_t leaf_count;
    uint32_t leaf_size;
    uint32_t tree;
    uint32_t vocab_chunk;
    uint32_t schedule;
} iso_contract;

/* Fill *c with the defaults above and the given leaf shape and vocab chunk.
 * Returns ISO_ERR_ARG for a NULL pointer; the result is not validated. */
iso_status iso_contract_init(iso_contract *c, uint32_t leaf_count, uint32_t leaf_size,
                             uint32_t vocab_chunk);

/* ISO_OK if *c is well formed (see the field list), else ISO_ERR_CONTRACT
 * (ISO_ERR_DTYPE for an unsupported dtype, ISO_ERR_ARG for NULL). */
iso_status iso_contract_validate(const iso_contract *c);

/*
 * numerical_policy identity ([AGL] "Contract Structure and Enforcement",
 * identities; [KTB] section 6, the contract digest as a lockfile):
 * out[32] = SHA-256 (FIPS 180-4) of the 24-byte tag
 * "iso.numerical_policy.v1" followed by one NUL byte, then the eight uint32
 * fields above in declaration order, little-endian (56 bytes in all).
 * The contract must validate first.  Host only; never touches the GPU.
 */
iso_status iso_contract_digest(const iso_contract *c, uint8_t out[32]);

/* ISO_OK if the digest of *c equals want[32], ISO_ERR_IDENTITY otherwise. */
iso_status iso_contract_check(const iso_contract *c, const uint8_t want[32]);

/*
 * Topology claim ([AGL] "Contract Structure and Enforcement", claims): a
 * contract with L leaves is proven partition-invariant for P in {1, 2, 4, 8}
 * with P dividing L.  Partition p owns the contiguous leaf block
 * [p*L/P, (p+1)*L/P), a whole subtree ([AGL] TP bullet: the contract fixes
 * the rank-to-leaf map).  Returns ISO_OK or ISO_ERR_CLAIM.
 */
iso_status iso_check_partitions(const iso_contract *c, int partitions);

/* ---------------------------------------------------------------- identities
 * [AGL] "Contract Structure and Enforcement": an execution contract splits
 * the forward operators into regions (arithmetic spans implemented by one
 * kernel) and cases (such as engine_prefill and trainer_fwd) saying how each
 * region runs; each (region, case) pair pins a composition (accumulation
 * dtype, reduction decomposition); claims list the partition counts for which
 * the tree is proven not to change the bits; SHA-256 identities named
 * semantic, numerical_policy and deployment let two runtimes check that they
 * run the same verified policy.  [KTB] section 6: a model checksum plus a
 * numerical-execution checksum, checked like a lockfile.
 */

/* SHA-256 over any bytes, fed in pieces.  The semantic identity is this
 * digest over the model's weights and configuration, in an order the caller
 * fixes.  Errors: ISO_ERR_ARG for NULL (update accepts n == 0 with NULL). */
typedef struct iso_sha256 {
    uint32_t h[8];
    uint64_t nbytes;
    uint8_t buf[64];
    uint32_t nbuf;
} iso_sha256;
iso_status iso_sha256_init(iso_sha256 *s);
iso_status iso_sha256_update(iso_sha256 *s, const void *data, size_t n);
iso_status iso_sha256_final(iso_sha256 *s, uint8_t out[32]);

/* One (region, case) composition of an execution contract.
 *   region, case_name  NUL-terminated ASCII names of 1..31 characters
 *                      (bytes after the NUL are ignored)
 *   policy             the region's contract, as passed to its entry point
 *   partitions         the partition count this case runs the region with
 *   claims             bit k set: partition count 2^k (k = 0..3) is claimed
 *                      not to change the region's bits; every claimed count
 *                      must divide the policy's leaf count (MFMA schedule)
 *                      or be 1 (sequential schedule) */
typedef struct iso_composition {
    char region[32];
    char case_name[32];
    iso_contract policy;
    uint32_t partitions;
    uint32_t claims;
} iso_composition;

/* numerical_policy and deployment identities of a table of n compositions
 * (each (region, case) at most once; the table's order does not matter):
 *   numerical_policy = SHA-256 of the 30-byte tag
 *       "iso.numerical_policy.table.v1\0", n as uint32 LE, then for every
 *       composition in (region, case_name) byte order: region and case_name
 *       zero-padded to 32 bytes each, the 8 policy fields and claims as
 *       uint32 LE;
 *   deployment = SHA-256 of the 18-byte tag "iso.deployment.v1\0",
 *       iso_version() zero-padded to 32 bytes, n as uint32 LE, then for
 *       every composition in the same order: region[32], case_name[32],
 *       partitions as uint32 LE.
 * Errors: ISO_ERR_ARG for NULL, a bad name or a repeated (region, case); a
 * malformed policy's own code; ISO_ERR_CLAIM when partitions is not claimed
 * or a claim is not a valid split of the policy. */
iso_status iso_table_digests(const iso_composition *table, size_t n,
                             uint8_t numerical_policy[32], uint8_t deployment[32]);

/* The per-call check before a launch: the (region, case) composition must be
 * in the table (ISO_ERR_ARG otherwise), `c` must have its policy's
 * numerical_policy digest (ISO_ERR_IDENTITY), and `partitions` must be
 * among its claims (ISO_ERR_CLAIM). */
iso_status iso_table_check(const iso_composition *table, size_t n, const char *region,
                           const char *case_name, const iso_contract *c, int partitions);

/* Workspace bytes iso_gemm can use for this shape (0 when none); (size_t)-1
 * for arguments iso_gemm would reject.  With P > 1 (or more than 16 leaves
 * per partition outside the few-rows kernel) the workspace is required.
 * With P = 1 on an output of fewer than 128 tiles of 128 x 128 and more
 * than 16 rows (more than 32 on a layer of at most 8 MiB of weights), the
 * size returned lets the call split K into up to eight (up to 64 rows) or
 * four (more rows) partitions of whole subtrees internally (same bits, more
 * workgroups); a call given less runs without that split. */
size_t iso_gemm_workspace(const iso_contract *c, int64_t M, int64_t N, int partitions);

/*
 * Invariant GEMM ([AGL] "Achieving Parallelism Invariance", TP bullet):
 *   C [M][N] = A [M][K] * W, W passed as Wt [N][K]; K = L * m.
 *   out_dtype ISO_F32: C is FP32, the tree root.
 *   out_dtype ISO_BF16: C is bf16, the FP32 root rounded to nearest-even.
 * `partitions` P emulates P tensor-parallel ranks on this GPU: partition p
 * computes its subtree root into the workspace and a combine kernel applies
 * the top log2(P) levels.  Every P allowed by the claim gives the same bits.
 * The launch shape follows the problem, never the numbers: 128 x 128 or
 * 128 x 256 tiles; with P = 1, for shapes the weight-streaming kernel takes
 * (4 or 8-64 leaves of 64-512 columns, K <= 4096), one workgroup per 16
 * output columns for up to 16 rows, up to 32 on a layer of at most 8 MiB of
 * weights or without a workspace, and up to 96 without the split below on
 * an output of fewer than 128 tiles with 8 or more leaves; with P = 1, a
 * workspace and fewer than 128 output tiles, an internal split of K (see
 * iso_gemm_workspace).  A row's bits do not depend on M, on its position,
 * or on which of these runs.
 * Limits: M, N < 2^23 and (M/128)(N/128) < 2^28 tiles, K <= 2^22.
 */
iso_status iso_gemm(const iso_contract *c, const void *A, const void *Wt, void *C,
                    uint32_t out_dtype, int64_t M, int64_t N, int64_t K, int partitions,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Non-invariant comparison profile ([KTB] section 20, correctness versus
 * performance profiles): the same tiles with ONE accumulator over all of K
 * (no leaves, no tree).  Its bits match iso_gemm's only by accident; it
 * exists to measure the cost of invariance.  Arguments as iso_gemm minus the
 * contract and partitions.  K: multiple of 64.
 */
iso_status iso_gemm_baseline(const void *A, const void *Wt, void *C, uint32_t out_dtype,
                             int64_t M, int64_t N, int64_t K, void *stream);

/* Workspace bytes iso_lmhead_logprob needs; (size_t)-1 for bad arguments. */
size_t iso_lmhead_workspace(const iso_contract *c, int64_t M, int64_t V, int partitions);

/*
 * Sampled-token logprob ([KTB] section 1: the rollout records the sampled
 * token's logprob and the trainer recomputes it; section 4: their ratio):
 *   z = H [M][K] * W_vocab, W_vocab passed as Wvt [V][K], FP32 logits from
 *       the same leaf/tree contraction as iso_gemm (never rounded to bf16,
 *       never written to memory);
 *   logprob[i] = z[i][t] - logsumexp(z[i][:]),  t = tok[i].
 * The softmax reduction is itself a fixed tree: the vocabulary is cut into
 * chunks of 128 ids; per chunk the max and the sum of exp(z - chunk max)
 * are reduced over a balanced binary tree in index order, and the chunk
 * pairs (m, s) are merged over the balanced tree in chunk order (padded with
 * the identity (-inf, 0)) by (m, s) + (m', s') = (u, s e^(m-u) + s' e^(m'-u)),
 * u = max(m, m').  c->vocab_chunk must be ISO_VOCAB_CHUNK.  A token id
 * outside [0, V) gives NaN for its row.  Up to 16 rows (one partition) run a
 * decode kernel that streams the vocabulary matrix once; the bits are those
 * of the same rows in any larger batch.  Limits: 1 <= V <= 2^20, M < 2^31.
 */
iso_status iso_lmhead_logprob(const iso_contract *c, const void *H, const void *Wvt,
                              const int32_t *tok, float *logprob, int64_t M, int64_t V,
                              int64_t K, int partitions, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * iso_lmhead_logprob for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same numbers, bit for bit, with the workspace taken from
 * a static device array of ISO_LMHEAD_NOALLOC_BYTES that the library holds
 * on every GPU it runs on until the process ends.  The call allocates and
 * frees nothing; the first call on a device looks up that device's copy.
 * One partition (arguments as iso_lmhead_logprob without partitions and
 * workspace).  A shape whose statistics (M * ceil(V / 128) * 8 bytes plus
 * M * 4, each rounded up to 256) exceed the scratch gives ISO_ERR_WORKSPACE
 * before any launch: at V = 151936 up to 3532 rows fit.  Every call on one
 * GPU shares the one scratch: calls that overlap on a GPU (two streams, two
 * threads) race and must be ordered by the caller.
 */
#define ISO_LMHEAD_NOALLOC_BYTES ((size_t)32 << 20)
iso_status iso_lmhead_logprob_noalloc(const iso_contract *c, const void *H, const void *Wvt,
                                      const int32_t *tok, float *logprob, int64_t M, int64_t V,
                                      int64_t K, void *stream);

/*
 * The vocabulary-sharded LM-head, split at its exchange point (one GPU
 * stands in for the ranks of a vocabulary-parallel layer; [AGL] "Achieving
 * Parallelism Invariance": partials are combined by the fixed tree whatever
 * the layout).  A shard owns the whole chunks of token ids [v_begin, v_end)
 * of a V-token vocabulary (v_begin a multiple of ISO_VOCAB_CHUNK; v_end too,
 * or v_end = V) and Wvt_shard points at row v_begin of Wvt [V][K].
 * iso_lmhead_shard_stats writes, for each row r and each chunk c of the
 * shard, stats[r][c][0] = the chunk max and stats[r][c][1] = the chunk's
 * exp-sum tree (both FP32, stats is [M][ceil(V / 128)][2]), and target[r] =
 * the FP32 logit of tok[r] when tok[r] lies in the shard.  Once every shard
 * has written (in any order: the writes are disjoint), iso_lmhead_finish
 * folds each row's chunk pairs over the balanced tree in chunk order and
 * gives the same logprob bits as iso_lmhead_logprob (NaN for a token id
 * outside [0, V)).  The contract is the iso_lmhead_logprob one, with at most
 * 16 leaves (the per-shard kernel runs one partition).  Buffers are the
 * caller's, device memory; a row's stats come only from its own data.
 */
iso_status iso_lmhead_shard_stats(const iso_contract *c, const void *H, const void *Wvt_shard,
                                  const int32_t *tok, float *stats, float *target, int64_t M,
                                  int64_t V, int64_t v_begin, int64_t v_end, int64_t K,
                                  void *stream);
iso_status iso_lmhead_finish(const float *stats, const float *target, const int32_t *tok,
                             float *logprob, int64_t M, int64_t V, void *stream);

/*
 * Batch-invariant RMSNorm with an optional residual add, the normalization
 * in front of the LM-head ([KTB] section 4: normalization is one of the
 * reductions whose order changes a row's bits; section 8: fix the reduction
 * tree instead of letting the layout choose it).  Per row of H elements:
 *   h   = bf16(x + residual) when residual != NULL (FP32 add, rounded to
 *         nearest even), else h = x; residual_out <- h when not NULL;
 *   ss  = the sum of h_i * h_i over the row: contiguous leaves of
 *         c->leaf_size elements, each summed one term at a time in ascending
 *         order in FP32, then the balanced tree over the c->leaf_count leaf
 *         sums (squares of bf16 values are exact in FP32);
 *   r   = 1 / sqrt(ss / H + eps), FP32, each operation correctly rounded;
 *   y_i = (h_i * r) * w_i in FP32, rounded to bf16 (out_dtype ISO_BF16) or
 *         kept (ISO_F32).
 * Every step is a correctly rounded FP32 operation in a fixed order, so a
 * row's bits depend only on that row, and a plain FP32 evaluation in the
 * same order reproduces them.  c->schedule must be ISO_SCHED_SEQ_KASC and
 * c->vocab_chunk 0.  Layouts: x, residual, residual_out bf16 [M][H]; weight
 * bf16 [H]; y [M][H] of out_dtype; all 16-byte aligned.  Limits: H = L * m;
 * S = H / min(L, 64) is 8, 16, 32, 64 or 128 and S / m is 1, 2, 4 or 8 (a
 * wave handles a row, each lane one leaf or L/64 whole leaves); M < 2^31;
 * eps finite and >= 0.  residual_out may alias residual (in place); y must
 * not alias an input and residual_out must not alias x (ISO_ERR_ARG).
 * Shape errors give ISO_ERR_SHAPE, a matrix-product contract ISO_ERR_CONTRACT.
 */
iso_status iso_rmsnorm(const iso_contract *c, const void *x, const void *residual,
                       void *residual_out, const void *weight, void *y, uint32_t out_dtype,
                       int64_t M, int64_t H, float eps, void *stream);

/*
 * CPR gated delta rule ([AGL] "Chunkwise-Parallel Recurrent (CPR) Gated
 * DeltaNet"; [KTB] sections 10-11): the recurrence is the numerical
 * definition, evaluated in parallel across chunks, and decode re-syncs the
 * state every C tokens so that prefill and decode give the same bits.  The
 * pages give no equations; the rule is, per head with a d x d FP32 state S
 * (row a = value index, column j = key index),
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 * one token step being u = S k, w = beta (v - alpha u), S <- alpha S + w k^T,
 * o = S q (dot products: balanced trees over the d products in index order;
 * every other operation one FP32 multiply or add, no contraction).  Inside
 * chunk c the outputs are token steps from the chunk's boundary state B_c;
 * the next boundary is B_{c+1} = U_c + B_c P_c, with (P_c, U_c) the chunk
 * form of the same map (backward scan R = I, U = 0; for i = C-1 .. 0:
 * r = k_i^T R, U <- U + (beta_i v_i) r, R <- alpha_i (R - (beta_i k_i) r);
 * P_c = R), not the stepped state.
 *
 * Contract: schedule ISO_SCHED_CPR_GDN, leaf_count = d (the kernels take 128),
 * leaf_size = C (1..64), vocab_chunk 0 (else ISO_ERR_CONTRACT; d != 128 is
 * ISO_ERR_SHAPE).  Layouts: q, k, v bf16 [T][H][d]; alpha, beta FP32
 * [T][H]; states FP32 [H][d][d] row-major; all 16-byte aligned.
 * Limits: 1 <= H < 65536, 0 <= T, ceil(T / C) < 65536.
 */

/* Workspace bytes iso_cpr_prefill needs for T tokens (pass T = C for
 * iso_cpr_decode_step); (size_t)-1 for arguments the calls would reject. */
size_t iso_cpr_workspace(const iso_contract *c, int64_t H, int64_t T);

/*
 * Prefill of T tokens from the boundary state S0 (NULL: zeros):
 *   o     FP32 [T][H][d]  outputs
 *   snap  FP32 [H][d][d]  B_{floor(T/C)}, the last boundary state
 *   run   FP32 [H][d][d]  the state the next decode step continues from:
 *                         snap when T is a multiple of C, else the stepped
 *                         state after token T-1
 * S0 may alias snap; snap and run must differ and o must not alias an input
 * (ISO_ERR_ARG).
 */
iso_status iso_cpr_prefill(const iso_contract *c, const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta, const float *S0, float *o,
                           float *snap, float *run, int64_t T, int64_t H, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * One decode step of token `pos` for every head.  q, k, v, alpha, beta are
 * the sequence arrays of the prefill layout holding tokens 0..pos (token pos
 * just appended); snap and run (FP32 [H][d][d], distinct) are updated in
 * place and o (FP32 [H][d]) receives the outputs.  When pos + 1 is a multiple
 * of C the step also re-syncs: snap and run become B_{(pos+1)/C} from the
 * chunk form of tokens pos-C+1 .. pos, which gives the same bits as a
 * prefill through pos.  Workspace: iso_cpr_workspace(c, H, C) bytes.
 */
iso_status iso_cpr_decode_step(const iso_contract *c, const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta, int64_t pos, float *snap,
                               float *run, float *o, int64_t H, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Byte offsets of the MoE workspace regions, for inspection of the stages.
 *   idx    int32 [T][top_k]   expert ids in routing order
 *   gate   float [T][top_k]   renormalised gates in routing order
 *   h      bf16  [T][top_k][I] SwiGLU activations
 *   e      float [T][top_k][H] expert outputs before the combine
 * The remaining bytes up to `total` hold the per-expert buckets and the
 * work list.  Returns ISO_ERR_ARG / ISO_ERR_SHAPE for arguments
 * iso_moe_combine would reject for those reasons. */
typedef struct iso_moe_layout {
    size_t idx, gate, h, e, total;
} iso_moe_layout;

iso_status iso_moe_layout_of(int64_t T, int64_t H, int64_t E, int64_t I, int top_k,
                             iso_moe_layout *out);

/* Workspace bytes iso_moe_combine needs; (size_t)-1 for bad arguments. */
size_t iso_moe_workspace(int64_t T, int64_t H, int64_t E, int64_t I, int top_k);

/*
 * MoE FFN with a fixed routing-order combine ([AGL] "Achieving Parallelism
 * Invariance", EP bullet: expert outputs are combined in a fixed routing
 * order rather than rank order; [KTB] section 9).
 *   route:   per token, softmax over E FP32 router logits; the top_k experts
 *            by (logit descending, expert id ascending) -- the routing
 *            order; gates = their probabilities renormalised to sum to one.
 *   experts: per (token, slot) with expert e: G = x Wg[e], U = x Wu[e]
 *            (gate_up contract, K = H), h = bf16(silu(G) * U),
 *            out = h Wd[e] (down contract, K = I), all FP32 leaf/tree GEMMs.
 *   combine: y = g_0 out_0, then y = y + g_k out_k for k = 1..top_k-1,
 *            FP32, each product rounded before its add.
 * Layouts: X bf16 [T][H]; router_logits float [T][E]; Wg, Wu bf16 [E][I][H];
 * Wd bf16 [E][H][I]; Y float [T][H].  Each token's bits do not depend on the
 * other tokens in the batch or their order.  Router logits must be finite.
 * Limits: 1 <= E <= 1024, 1 <= top_k <= min(16, E), leaf_count <= 16 in both
 * contracts, T * top_k < 2^31, T * H * 2 and T * top_k * I * 2 below 2^32
 * bytes.  X, the weights and Y must be 16-byte aligned.
 */
iso_status iso_moe_combine(const iso_contract *gate_up, const iso_contract *down,
                           const void *X, const float *router_logits, const void *Wg,
                           const void *Wu, const void *Wd, float *Y, int64_t T, int64_t H,
                           int64_t E, int64_t I, int top_k, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * The expert FFN's activation on its own (the SwiGLU step of
 * iso_moe_combine; [AGL] "Achieving Parallelism Invariance", EP bullet: the
 * expert computations are part of the invariant region), for a dense FFN
 * built from iso_gemm calls and for checking the MoE stage by stage:
 *   h[i]   = bf16(silu(G[i]) * U[i]), rounded to nearest even;
 *   act[i] = silu(G[i]) * U[i] in FP32 before that rounding (act may be NULL);
 * silu(g) = g / (1 + e^-g), FP32, e^-g on the hardware exp2 of -g log2(e).
 * It is the same device function as the MoE gate/up epilogue, so G and U
 * with the bits of that stage (iso_gemm with the gate_up contract gives
 * them) reproduce its h bit for bit.  G, U, act: FP32 [n]; h: bf16 [n];
 * device memory, no alignment needed; act and h must not overlap G or U.
 * n == 0 returns ISO_OK; n < 0 or a NULL G, U or h gives ISO_ERR_ARG.
 */
iso_status iso_swiglu(const float *G, const float *U, float *act, void *h, int64_t n,
                      void *stream);

/* Static description of a status code. */
const char *iso_status_str(iso_status s);

/* Library version string, e.g. "iso 0.1.0 gfx950". */
const char *iso_version(void);

/* The HIP runtime's description of the last launch result of an entry point
 * on the calling thread ("no error" after a successful launch). */
const char *iso_last_launch_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ISO_H_ */
