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
