/*
 * iso_oracle.c -- plain, slow, obviously correct CPU oracle for the
 * parallelism- and batch-invariant numerics path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or constant with the HIP
 * library: the two meet only in the seeded input bit patterns.
 *
 * Pages cited (web pages about IsoExec):
 *   [AGL] "IsoExec: Eliminating Trainer-Inference Mismatch in SkyRL"
 *         (agentlenshq.com blog summary)
 *   [KTB] katelyatop-blog.pages.dev post on vLLM/SkyRL IsoExec and the
 *         trainer-inference mismatch (numbered sections)
 *   [DDV] "IsoExec: Unified Execution to Eliminate Trainer-Inference
 *         Mismatch in SkyRL" (daily.dev summary)
 *
 * What is computed, and the readings taken where the pages are silent:
 *
 *  GEMM  C = A * W, with A [M][K] bf16 and W given as its transpose Wt
 *        [N][K] bf16.  [AGL] "Achieving Parallelism Invariance", TP bullet:
 *        K is cut into contiguous leaves, each leaf is a dot product with FP32
 *        accumulation, and the partials are combined by a fixed binary
 *        reduction tree ([KTB] section 8 shows (A+B)+(C+D) for four partials).
 *        Readings: leaves are equal, K = L*m; inside a leaf the products are
 *        added one at a time in ascending k (the pages leave the in-leaf order
 *        to the hardware; the oracle's own order is the plain sequential sum);
 *        the tree is the balanced one over leaf index, pairing (2i, 2i+1) at
 *        every level.  bf16*bf16 products are exact in FP32.
 *
 *  PARTITIONS  [AGL] same bullet: the contract fixes the rank-to-leaf map.
 *        Reading: partition p of P owns the contiguous leaf block
 *        [p*L/P, (p+1)*L/P), i.e. one whole subtree; the P subtree roots are
 *        then combined by the top log2(P) levels of the same tree.
 *
 *  LOGPROB  [KTB] section 1 (rollout records the sampled token's logprob, the
 *        trainer recomputes it) and section 4 (ratio of the two).  The value is
 *        the plain definition log softmax(z)[t] = z_t - max z - log sum exp(z -
 *        max z), evaluated in float64 from the FP32 logits z of the GEMM above.
 *
 *  MOE   [AGL] EP bullet and [KTB] section 9: expert outputs are combined in a
 *        fixed routing order, never in rank or completion order.  Readings:
 *        gate probabilities are a softmax over all experts, the top_k experts
 *        are taken by (logit descending, expert id ascending) and that is the
 *        routing order; the k gates are renormalised to sum to one; the expert
 *        FFN is SwiGLU, h = silu(x Wg) * (x Wu), with h rounded to bf16 (the
 *        down projection is again a bf16 leaf GEMM); y = sum_k g_k * e_k.
 *        Softmax, gates and the final combine are evaluated in float64 (plain
 *        definition); the three GEMMs follow the FP32 leaf/tree order above;
 *        silu is float64 rounded to float32, and the bf16 rounding of h is
 *        decided on the FP32 product silu(G)*U, the precision the kernel takes
 *        that decision in.
 *
 *  RMSNORM  [KTB] section 4 names normalization among the reductions whose
 *        order changes a row's result; section 8 fixes the reduction tree.
 *        The pages give no formula, so the reading is the common RMSNorm
 *        with a residual add in front: h = bf16(x + r), y_i = h_i /
 *        sqrt(mean_i(h_i^2) + eps) * w_i.  The sum of squares follows the
 *        same leaf/tree reading as the GEMM (contiguous leaves, sequential
 *        FP32 in-leaf sums, balanced tree over the leaves); the mean, the
 *        square root and the reciprocal are single FP32 operations; the scale
 *        is applied as (h_i * r) * w_i.
 *
 *  CPR   [AGL] "Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet" and [KTB]
 *        sections 10-11: the recurrence is the primary numerical definition,
 *        evaluated in parallel across chunks, and decode re-synchronises the
 *        hidden state every C tokens (C = chunk size), so trainer, prefill and
 *        decode agree bit for bit.  The pages give no GDN equations; the reading
 *        is the gated delta rule with a d x d state S (row a = value index,
 *        column j = key index) per head:
 *            S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *            o_t = S_t q_t,
 *        one token "step" evaluated as u = S k, w = beta (v - alpha u),
 *        S <- alpha S + w k^T, o = S q, each dot product a balanced binary tree
 *        over the d products in index order, every other operation a single
 *        FP32 multiply or add in the order written.  CPR reading: inside chunk
 *        c every output comes from steps started at the chunk's boundary state
 *        B_c; the next boundary state is not the stepped state but the chunk
 *        form of the same map, B_{c+1} = B_c P_c + U_c with P_c = A_0 ... A_{C-1}
 *        (A_i = alpha_i (I - beta_i k_i k_i^T)) and U_c = sum_i beta_i v_i k_i^T
 *        A_{i+1} ... A_{C-1}, both built by a backward scan over the chunk that
 *        needs no state; the pass B_c -> B_{c+1} is a d x d x d product with
 *        tree-ordered sums.  A decode step is the same token step on the
 *        running state; when a token closes a chunk the running state is
 *        replaced by B_{c+1} from the same chunk form (the re-sync).
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * OpenMP splits independent output rows only; no element's order changes.
 * All entry points return 0 on success and -1 on bad arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- helpers */

static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a finite float to bf16, nearest with ties to even. */
static uint16_t float_to_bf16_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u = u + 0x7FFFu + keep_lsb;
    return (uint16_t)(u >> 16);
}

static int is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the following calls (n >= 1); no effect on any result,
 * since threads only split independent outputs. */
int oracle_set_threads(int n)
{
    if (n < 1)
        return -1;
#ifdef _OPENMP
    omp_set_num_threads(n);
#endif
    return 0;
}

/* One leaf: sequential FP32 sum over k in [k0, k1), ascending. */
static float leaf_dot(const float *a, const uint16_t *w, int64_t k0, int64_t k1)
{
    float s = 0.0f;
    for (int64_t k = k0; k < k1; ++k) {
        float prod = a[k] * bf16_bits_to_float(w[k]); /* exact for bf16 inputs */
        s = s + prod;
    }
    return s;
}

/* Balanced binary tree over v[0..n), n a power of two, in index order:
 * each level replaces v[i] by v[2i] + v[2i+1].  Returns the root. */
static float tree_fold(float *v, int n)
{
    for (int width = n; width > 1; width /= 2)
        for (int i = 0; i < width / 2; ++i)
            v[i] = v[2 * i] + v[2 * i + 1];
    return v[0];
}

/* Contract dot product of one A row (already widened) with one stored weight
 * row: L leaves of m = K/L, each a sequential sum, then the balanced tree. */
static float contract_dot(const float *a, const uint16_t *w, int64_t K, int L, float *leaf)
{
    int64_t m = K / L;
    for (int l = 0; l < L; ++l)
        leaf[l] = leaf_dot(a, w, (int64_t)l * m, (int64_t)(l + 1) * m);
    return tree_fold(leaf, L);
}

static int gemm_args_ok(int64_t M, int64_t N, int64_t K, int L)
{
    return M >= 0 && N >= 0 && K > 0 && is_pow2(L) && K % L == 0;
}

/* ------------------------------------------------------------------- GEMM */

/* C[i][j] (FP32) = contract dot of A row i with Wt row j. */
int oracle_gemm(const uint16_t *A, const uint16_t *Wt, int64_t M, int64_t N, int64_t K,
                int L, float *C)
{
    if (!gemm_args_ok(M, N, K, L) || !A || !Wt || !C)
        return -1;
#pragma omp parallel
    {
        float *a = (float *)malloc((size_t)K * sizeof(float));
        float *leaf = (float *)malloc((size_t)L * sizeof(float));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t k = 0; k < K; ++k)
                a[k] = bf16_bits_to_float(A[i * K + k]);
            for (int64_t j = 0; j < N; ++j)
                C[i * N + j] = contract_dot(a, Wt + j * K, K, L, leaf);
        }
        free(leaf);
        free(a);
    }
    return 0;
}

/* Selected elements only: out[q] = C[rows[q]][cols[q]]. */
int oracle_gemm_elems(const uint16_t *A, const uint16_t *Wt, int64_t K, int L,
                      const int64_t *rows, const int64_t *cols, int64_t n, float *out)
{
    if (!gemm_args_ok(1, 1, K, L) || n < 0 || !A || !Wt || !rows || !cols || !out)
        return -1;
#pragma omp parallel
    {
        float *a = (float *)malloc((size_t)K * sizeof(float));
        float *leaf = (float *)malloc((size_t)L * sizeof(float));
#pragma omp for schedule(dynamic, 16)
        for (int64_t q = 0; q < n; ++q) {
            for (int64_t k = 0; k < K; ++k)
                a[k] = bf16_bits_to_float(A[rows[q] * K + k]);
            out[q] = contract_dot(a, Wt + cols[q] * K, K, L, leaf);
        }
        free(leaf);
        free(a);
    }
    return 0;
}

/* Rank emulation: partition p computes the subtree over its own contiguous
 * leaf block, then the P roots go through the remaining tree levels.  Used to
 * check that the oracle's own tree is partition-invariant. */
int oracle_gemm_partitioned(const uint16_t *A, const uint16_t *Wt, int64_t M, int64_t N,
                            int64_t K, int L, int P, float *C)
{
    if (!gemm_args_ok(M, N, K, L) || !is_pow2(P) || P > L || !A || !Wt || !C)
        return -1;
    int64_t m = K / L;
    int per = L / P;
#pragma omp parallel
    {
        float *a = (float *)malloc((size_t)K * sizeof(float));
        float *leaf = (float *)malloc((size_t)per * sizeof(float));
        float *root = (float *)malloc((size_t)P * sizeof(float));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t k = 0; k < K; ++k)
                a[k] = bf16_bits_to_float(A[i * K + k]);
            for (int64_t j = 0; j < N; ++j) {
                const uint16_t *w = Wt + j * K;
                for (int p = 0; p < P; ++p) {
                    for (int l = 0; l < per; ++l) {
                        int64_t gl = (int64_t)p * per + l;
                        leaf[l] = leaf_dot(a, w, gl * m, (gl + 1) * m);
                    }
                    root[p] = tree_fold(leaf, per);
                }
                C[i * N + j] = tree_fold(root, P);
            }
        }
        free(root);
        free(leaf);
        free(a);
    }
    return 0;
}

/* ---------------------------------------------------------------- logprob */

/* Log-probability of token tok[i] under softmax of row i's logits, where the
 * logits are the FP32 contract GEMM of H row i with every vocabulary row of
 * Wvt [V][K].  Optional outputs: the target logit (FP32) and the row's
 * log-sum-exp (float64).  A token id outside [0, V) gives NaN. */
int oracle_lmhead_logprob(const uint16_t *H, const uint16_t *Wvt, const int32_t *tok,
                          int64_t M, int64_t V, int64_t K, int L, double *logprob,
                          float *z_target, double *lse)
{
    if (!gemm_args_ok(M, V, K, L) || V < 1 || !H || !Wvt || !tok || !logprob)
        return -1;
#pragma omp parallel
    {
        float *a = (float *)malloc((size_t)K * sizeof(float));
        float *leaf = (float *)malloc((size_t)L * sizeof(float));
        float *z = (float *)malloc((size_t)V * sizeof(float));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t k = 0; k < K; ++k)
                a[k] = bf16_bits_to_float(H[i * K + k]);
            double zmax = -INFINITY;
            for (int64_t j = 0; j < V; ++j) {
                z[j] = contract_dot(a, Wvt + j * K, K, L, leaf);
                if (z[j] > zmax)
                    zmax = z[j];
            }
            double sum = 0.0;
            for (int64_t j = 0; j < V; ++j)
                sum += exp((double)z[j] - zmax);
            double l = zmax + log(sum);
            int64_t t = tok[i];
            if (t < 0 || t >= V) {
                logprob[i] = NAN;
                if (z_target)
                    z_target[i] = NAN;
            } else {
                logprob[i] = ((double)z[t] - zmax) - log(sum);
                if (z_target)
                    z_target[i] = z[t];
            }
            if (lse)
                lse[i] = l;
        }
        free(z);
        free(leaf);
        free(a);
    }
    return 0;
}

/* -------------------------------------------------------------------- MoE */

/* Routing: idx[t][k] = k-th expert by (logit descending, id ascending);
 * gate[t][k] = softmax probability of that expert divided by the sum of the
 * selected top_k probabilities (float64). */
int oracle_moe_route(const float *logits, int64_t T, int64_t E, int top_k, int32_t *idx,
                     double *gate)
{
    if (T < 0 || E < 1 || top_k < 1 || top_k > E || !logits || !idx || !gate)
        return -1;
#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)E * sizeof(double));
        unsigned char *taken = (unsigned char *)malloc((size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const float *l = logits + t * E;
            double mx = -INFINITY;
            for (int64_t e = 0; e < E; ++e)
                if (l[e] > mx)
                    mx = l[e];
            double z = 0.0;
            for (int64_t e = 0; e < E; ++e) {
                p[e] = exp((double)l[e] - mx);
                z += p[e];
            }
            for (int64_t e = 0; e < E; ++e)
                p[e] /= z;
            memset(taken, 0, (size_t)E);
            double psel = 0.0;
            for (int k = 0; k < top_k; ++k) {
                int64_t best = -1;
                for (int64_t e = 0; e < E; ++e) {
                    if (taken[e])
                        continue;
                    /* strictly greater keeps the lowest id among equal logits */
                    if (best < 0 || l[e] > l[best])
                        best = e;
                }
                taken[best] = 1;
                idx[t * top_k + k] = (int32_t)best;
                psel += p[best];
            }
            for (int k = 0; k < top_k; ++k)
                gate[t * top_k + k] = p[idx[t * top_k + k]] / psel;
        }
        free(taken);
        free(p);
    }
    return 0;
}

/* Gate/up projections and SwiGLU for every (token, slot):
 *   G = contract dot(x_t, Wg[e]), U = contract dot(x_t, Wu[e]) (FP32, L leaves)
 *   s = silu(G) in float64 rounded to FP32,  act = fl32(s * U),  h = bf16(act).
 * Wg, Wu are stored [E][I][H] (K = H contiguous).  act and h are [T][top_k][I]. */
int oracle_moe_gate_up(const uint16_t *X, const uint16_t *Wg, const uint16_t *Wu,
                       const int32_t *idx, int64_t T, int64_t Hd, int64_t E, int64_t I,
                       int top_k, int L, float *act, uint16_t *h)
{
    if (!gemm_args_ok(T, I, Hd, L) || E < 1 || top_k < 1 || !X || !Wg || !Wu || !idx || !h)
        return -1;
#pragma omp parallel
    {
        float *a = (float *)malloc((size_t)Hd * sizeof(float));
        float *leaf = (float *)malloc((size_t)L * sizeof(float));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t k = 0; k < Hd; ++k)
                a[k] = bf16_bits_to_float(X[t * Hd + k]);
            for (int s = 0; s < top_k; ++s) {
                int64_t e = idx[t * top_k + s];
                const uint16_t *wg = Wg + e * I * Hd;
                const uint16_t *wu = Wu + e * I * Hd;
                for (int64_t j = 0; j < I; ++j) {
                    float g = contract_dot(a, wg + j * Hd, Hd, L, leaf);
                    float u = contract_dot(a, wu + j * Hd, Hd, L, leaf);
                    float sg = (float)((double)g / (1.0 + exp(-(double)g)));
                    float v = sg * u;
                    int64_t o = (t * top_k + s) * I + j;
                    if (act)
                        act[o] = v;
                    h[o] = float_to_bf16_bits(v);
                }
            }
        }
        free(leaf);
        free(a);
    }
    return 0;
}

/* Down projection: e[t][k] = contract dot(h[t][k], Wd[e]) (FP32, L leaves).
 * Wd is stored [E][H][I] (K = I contiguous); h is [T][top_k][I]; e is
 * [T][top_k][H]. */
int oracle_moe_down(const uint16_t *h, const uint16_t *Wd, const int32_t *idx, int64_t T,
                    int64_t Hd, int64_t E, int64_t I, int top_k, int L, float *eout)
{
    if (!gemm_args_ok(T, Hd, I, L) || E < 1 || top_k < 1 || !h || !Wd || !idx || !eout)
        return -1;
#pragma omp parallel
    {
        float *a = (float *)malloc((size_t)I * sizeof(float));
        float *leaf = (float *)malloc((size_t)L * sizeof(float));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            for (int s = 0; s < top_k; ++s) {
                int64_t row = t * top_k + s;
                int64_t e = idx[row];
                for (int64_t k = 0; k < I; ++k)
                    a[k] = bf16_bits_to_float(h[row * I + k]);
                const uint16_t *wd = Wd + e * Hd * I;
                for (int64_t j = 0; j < Hd; ++j)
                    eout[row * Hd + j] = contract_dot(a, wd + j * I, I, L, leaf);
            }
        }
        free(leaf);
        free(a);
    }
    return 0;
}

/* Combine: y[t] = sum over k of gate[t][k] * e[t][k] (float64). */
int oracle_moe_combine(const double *gate, const float *eout, int64_t T, int64_t Hd, int top_k,
                       double *y)
{
    if (T < 0 || Hd < 1 || top_k < 1 || !gate || !eout || !y)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t j = 0; j < Hd; ++j) {
            double acc = 0.0;
            for (int k = 0; k < top_k; ++k)
                acc += gate[t * top_k + k] * (double)eout[(t * top_k + k) * Hd + j];
            y[t * Hd + j] = acc;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- RMSNORM */

/* Per row i of x [M][H] (bf16 bits): h = bf16(x + res) if res, else x
 * (written to res_out when given); ss = balanced tree over L leaves of
 * H / L, each the sequential FP32 sum of h_j * h_j; r = 1 / sqrtf(ss / H +
 * eps); y = (h_j * r) * w_j as float (out_bf16 = 0) or bf16 bits.  ss_out
 * (may be NULL) receives ss per row. */
int oracle_rmsnorm(const uint16_t *x, const uint16_t *res, const uint16_t *w, int64_t M,
                   int64_t H, int L, float eps, int out_bf16, uint16_t *res_out, void *y,
                   float *ss_out)
{
    if (M < 0 || H <= 0 || !is_pow2(L) || H % L != 0 || !x || !w || !y)
        return -1;
    const int64_t m = H / L;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t i = 0; i < M; ++i) {
        float *h = malloc((size_t)H * sizeof(float));
        float *leaf = malloc((size_t)L * sizeof(float));
        if (!h || !leaf) {
            bad = 1;
            free(h);
            free(leaf);
            continue;
        }
        for (int64_t j = 0; j < H; ++j) {
            float v = bf16_bits_to_float(x[i * H + j]);
            if (res) {
                uint16_t hb = float_to_bf16_bits(v + bf16_bits_to_float(res[i * H + j]));
                v = bf16_bits_to_float(hb);
            }
            h[j] = v;
            if (res_out)
                res_out[i * H + j] = float_to_bf16_bits(v); /* exact: v is a bf16 value */
        }
        for (int l = 0; l < L; ++l) {
            float s = 0.0f;
            for (int64_t j = l * m; j < (l + 1) * m; ++j)
                s = s + h[j] * h[j];
            leaf[l] = s;
        }
        const float ss = tree_fold(leaf, L);
        if (ss_out)
            ss_out[i] = ss;
        const float ms = ss / (float)H;
        const float r = 1.0f / sqrtf(ms + eps);
        for (int64_t j = 0; j < H; ++j) {
            const float v = (h[j] * r) * bf16_bits_to_float(w[j]);
            if (out_bf16)
                ((uint16_t *)y)[i * H + j] = float_to_bf16_bits(v);
            else
                ((float *)y)[i * H + j] = v;
        }
        free(h);
        free(leaf);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ CPR */

/* Balanced binary tree over x[0..d) * y[0..d) (d a power of two), products
 * rounded first, then pairs (2i, 2i+1) at every level. */
static float tree_dot(const float *x, const float *y, int d, float *tmp)
{
    for (int j = 0; j < d; ++j)
        tmp[j] = x[j] * y[j];
    return tree_fold(tmp, d);
}

/* One token of the gated delta rule on S [d][d]; writes o [d]. */
static void cpr_step(float *S, const float *q, const float *k, const float *v, float alpha,
                     float beta, int d, float *o, float *tmp)
{
    for (int a = 0; a < d; ++a) {
        float *row = S + (int64_t)a * d;
        const float u = tree_dot(row, k, d, tmp);
        const float w = beta * (v[a] - alpha * u);
        for (int j = 0; j < d; ++j)
            row[j] = alpha * row[j] + w * k[j];
        o[a] = tree_dot(row, q, d, tmp);
    }
}

/* Chunk form of n tokens (k, v [n][d] widened, alpha, beta [n]): the backward
 * scan R <- A_i R from R = I, U <- U + beta_i v_i (k_i^T R) before each update. */
static void cpr_transition(const float *k, const float *v, const float *alpha, const float *beta,
                           int n, int d, float *P, float *U, float *r, float *col, float *tmp)
{
    for (int m = 0; m < d; ++m)
        for (int j = 0; j < d; ++j)
            P[(int64_t)m * d + j] = m == j ? 1.0f : 0.0f;
    memset(U, 0, (size_t)d * d * sizeof(float));
    for (int i = n - 1; i >= 0; --i) {
        const float *ki = k + (int64_t)i * d, *vi = v + (int64_t)i * d;
        for (int j = 0; j < d; ++j) {
            for (int m = 0; m < d; ++m)
                col[m] = P[(int64_t)m * d + j];
            r[j] = tree_dot(ki, col, d, tmp);
        }
        for (int a = 0; a < d; ++a) {
            const float t = beta[i] * vi[a];
            for (int j = 0; j < d; ++j)
                U[(int64_t)a * d + j] = U[(int64_t)a * d + j] + t * r[j];
        }
        for (int m = 0; m < d; ++m) {
            const float sm = beta[i] * ki[m];
            for (int j = 0; j < d; ++j)
                P[(int64_t)m * d + j] = alpha[i] * (P[(int64_t)m * d + j] - sm * r[j]);
        }
    }
}

/* B_next = U + B P, every entry's sum over m a balanced tree. */
static void cpr_pass(const float *B, const float *P, const float *U, int d, float *Bn, float *col,
                     float *tmp)
{
    for (int j = 0; j < d; ++j) {
        for (int m = 0; m < d; ++m)
            col[m] = P[(int64_t)m * d + j];
        for (int a = 0; a < d; ++a)
            Bn[(int64_t)a * d + j] = U[(int64_t)a * d + j] + tree_dot(B + (int64_t)a * d, col, d, tmp);
    }
}

static void widen(const uint16_t *src, int64_t stride, int d, float *dst)
{
    for (int j = 0; j < d; ++j)
        dst[j] = bf16_bits_to_float(src[(int64_t)j * stride]);
    (void)stride;
}

/* Per-head scratch for the CPR entry points. */
struct cpr_scratch {
    float *q, *k, *v, *al, *be, *P, *U, *r, *col, *tmp, *o;
};
static int cpr_scratch_alloc(struct cpr_scratch *w, int C, int d)
{
    w->q = malloc((size_t)d * sizeof(float));
    w->k = malloc((size_t)C * d * sizeof(float));
    w->v = malloc((size_t)C * d * sizeof(float));
    w->al = malloc((size_t)C * sizeof(float));
    w->be = malloc((size_t)C * sizeof(float));
    w->P = malloc((size_t)d * d * sizeof(float));
    w->U = malloc((size_t)d * d * sizeof(float));
    w->r = malloc((size_t)d * sizeof(float));
    w->col = malloc((size_t)d * sizeof(float));
    w->tmp = malloc((size_t)d * sizeof(float));
    w->o = malloc((size_t)d * sizeof(float));
    return w->q && w->k && w->v && w->al && w->be && w->P && w->U && w->r && w->col && w->tmp && w->o;
}
static void cpr_scratch_free(struct cpr_scratch *w)
{
    free(w->q); free(w->k); free(w->v); free(w->al); free(w->be); free(w->P);
    free(w->U); free(w->r); free(w->col); free(w->tmp); free(w->o);
}

/* Token t of head h from [T][H][d] bf16 arrays, widened into k/v slot `slot`. */
static void cpr_load(const uint16_t *k, const uint16_t *v, const float *alpha, const float *beta,
                     int64_t H, int d, int64_t t, int64_t h, struct cpr_scratch *w, int slot)
{
    widen(k + (t * H + h) * d, 1, d, w->k + (int64_t)slot * d);
    widen(v + (t * H + h) * d, 1, d, w->v + (int64_t)slot * d);
    w->al[slot] = alpha[t * H + h];
    w->be[slot] = beta[t * H + h];
}

/*
 * Prefill of T tokens, H heads, head size d (a power of two), chunk C.
 *   q, k, v    [T][H][d] bf16 bits;  alpha, beta [T][H] FP32
 *   S0         [H][d][d] initial boundary state, or NULL for zeros
 *   o          [T][H][d] FP32 outputs
 *   snap       [H][d][d] the boundary state at the last chunk boundary <= T
 *   run        [H][d][d] the state a decode step continues from: the
 *              boundary state when T is a multiple of C, else the stepped
 *              state after token T-1
 *   bounds     optional [T/C + 1][H][d][d]: every boundary state B_0 .. B_{T/C}
 */
int oracle_cpr_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *alpha,
                       const float *beta, const float *S0, int64_t T, int64_t H, int d, int C,
                       float *o, float *snap, float *run, float *bounds)
{
    if (T < 0 || H <= 0 || !is_pow2(d) || C <= 0 || !q || !k || !v || !alpha || !beta || !o ||
        !snap || !run)
        return -1;
    const int64_t dd = (int64_t)d * d;
    const int64_t nb = T / C;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int64_t h = 0; h < H; ++h) {
        struct cpr_scratch w;
        float *B = malloc((size_t)dd * sizeof(float));
        float *Bn = malloc((size_t)dd * sizeof(float));
        float *S = malloc((size_t)dd * sizeof(float));
        if (!cpr_scratch_alloc(&w, C, d) || !B || !Bn || !S) {
            bad = 1;
            cpr_scratch_free(&w); free(B); free(Bn); free(S);
            continue;
        }
        if (S0)
            memcpy(B, S0 + h * dd, (size_t)dd * sizeof(float));
        else
            memset(B, 0, (size_t)dd * sizeof(float));
        if (bounds)
            memcpy(bounds + h * dd, B, (size_t)dd * sizeof(float));
        for (int64_t c0 = 0; c0 < T; c0 += C) {
            const int n = (int)(T - c0 < C ? T - c0 : C);
            memcpy(S, B, (size_t)dd * sizeof(float));
            for (int i = 0; i < n; ++i) {
                const int64_t t = c0 + i;
                cpr_load(k, v, alpha, beta, H, d, t, h, &w, i);
                widen(q + (t * H + h) * d, 1, d, w.q);
                cpr_step(S, w.q, w.k + (int64_t)i * d, w.v + (int64_t)i * d, w.al[i], w.be[i], d,
                         o + (t * H + h) * d, w.tmp);
            }
            if (n == C) {
                cpr_transition(w.k, w.v, w.al, w.be, n, d, w.P, w.U, w.r, w.col, w.tmp);
                cpr_pass(B, w.P, w.U, d, Bn, w.col, w.tmp);
                memcpy(B, Bn, (size_t)dd * sizeof(float));
                if (bounds)
                    memcpy(bounds + ((c0 / C + 1) * H + h) * dd, B, (size_t)dd * sizeof(float));
            }
        }
        memcpy(snap + h * dd, B, (size_t)dd * sizeof(float));
        memcpy(run + h * dd, (T % C == 0) ? B : S, (size_t)dd * sizeof(float));
        cpr_scratch_free(&w); free(B); free(Bn); free(S);
    }
    (void)nb;
    return bad ? -1 : 0;
}

/*
 * One decode step: token `pos` (q, k, v, alpha, beta hold tokens 0..pos in the
 * prefill layout), snap/run [H][d][d] in/out, o [H][d].  When pos closes a
 * chunk, snap and run both become the next boundary state (the re-sync).
 */
int oracle_cpr_decode_step(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const float *alpha, const float *beta, int64_t pos, int64_t H, int d,
                           int C, float *snap, float *run, float *o)
{
    if (pos < 0 || H <= 0 || !is_pow2(d) || C <= 0 || !q || !k || !v || !alpha || !beta || !snap ||
        !run || !o)
        return -1;
    const int64_t dd = (int64_t)d * d;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t h = 0; h < H; ++h) {
        struct cpr_scratch w;
        float *Bn = malloc((size_t)dd * sizeof(float));
        if (!cpr_scratch_alloc(&w, C, d) || !Bn) {
            bad = 1;
            cpr_scratch_free(&w); free(Bn);
            continue;
        }
        const int slot = (int)(pos % C);
        cpr_load(k, v, alpha, beta, H, d, pos, h, &w, slot);
        widen(q + (pos * H + h) * d, 1, d, w.q);
        cpr_step(run + h * dd, w.q, w.k + (int64_t)slot * d, w.v + (int64_t)slot * d, w.al[slot],
                 w.be[slot], d, o + h * d, w.tmp);
        if (slot == C - 1) {
            for (int i = 0; i < C; ++i)
                cpr_load(k, v, alpha, beta, H, d, pos - (C - 1) + i, h, &w, i);
            cpr_transition(w.k, w.v, w.al, w.be, C, d, w.P, w.U, w.r, w.col, w.tmp);
            cpr_pass(snap + h * dd, w.P, w.U, d, Bn, w.col, w.tmp);
            memcpy(snap + h * dd, Bn, (size_t)dd * sizeof(float));
            memcpy(run + h * dd, Bn, (size_t)dd * sizeof(float));
        }
        cpr_scratch_free(&w); free(Bn);
    }
    return bad ? -1 : 0;
}

/* The chunk form alone, for pins: P, U [d][d] of n tokens of one head
 * (k, v [n][d] bf16 bits, alpha, beta [n]). */
int oracle_cpr_transition(const uint16_t *k, const uint16_t *v, const float *alpha,
                          const float *beta, int n, int d, float *P, float *U)
{
    if (n <= 0 || !is_pow2(d) || !k || !v || !alpha || !beta || !P || !U)
        return -1;
    struct cpr_scratch w;
    if (!cpr_scratch_alloc(&w, n, d)) {
        cpr_scratch_free(&w);
        return -1;
    }
    for (int i = 0; i < n; ++i) {
        widen(k + (int64_t)i * d, 1, d, w.k + (int64_t)i * d);
        widen(v + (int64_t)i * d, 1, d, w.v + (int64_t)i * d);
        w.al[i] = alpha[i];
        w.be[i] = beta[i];
    }
    cpr_transition(w.k, w.v, w.al, w.be, n, d, P, U, w.r, w.col, w.tmp);
    cpr_scratch_free(&w);
    return 0;
}
