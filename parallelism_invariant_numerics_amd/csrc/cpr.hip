// cpr.hip -- chunkwise-parallel recurrent (CPR) gated delta rule for gfx950.
//
// "IsoExec: Eliminating Trainer-Inference Mismatch in SkyRL" (agentlenshq),
// section "Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet": the
// recurrence is the numerical definition, evaluated in parallel across
// chunks, and decode re-synchronises the hidden state every C tokens, so
// trainer, prefill and decode give the same bits.  The pages give no GDN
// equations; the gated delta rule used here is, per head with a d x d state S
// (row a = value index, column j = key index):
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.
//
// One token step: u = S k, w = beta (v - alpha u), S <- alpha S + w k^T,
// o = S q.  Every dot product is the balanced binary tree over the d = 128
// products in index order (64 per lane, the two halves joined across a lane
// pair), every other operation is one FP32 multiply or add in the order
// written (no contraction), so the bits are those of a plain FP32
// evaluation in the same order.
//
// CPR split, per head:
//   chunk form   (P_c, U_c) of chunk c from its tokens alone, by the backward
//                scan R = I, U = 0; for i = C-1 .. 0: r = k_i^T R,
//                U <- U + (beta_i v_i) r, R <- alpha_i (R - (beta_i k_i) r);
//                P_c = R.  All chunks in parallel.
//   pass         B_{c+1} = U_c + B_c P_c (tree-ordered sums over the 128
//                terms), sequential over chunks, parallel over state rows
//                (a row of B_{c+1} needs only the same row of B_c).
//   outputs      the token steps of chunk c started from B_c, all chunks in
//                parallel.
//   decode       the same token step on the running state; a token that
//                closes a chunk replaces the running state by B_{c+1} from
//                the chunk form (the re-sync), exactly as prefill does.
//
// Layouts: q, k, v [T][H][128] bf16; alpha, beta [T][H] FP32; states
// [H][128][128] FP32 row-major; P, U, boundary states [chunk][H][128][128].
#include "device_common.hpp"
#include "kernels.h"

namespace iso {

constexpr int kCprD = 128;
constexpr int kCprThreads = 256;
constexpr int kCprMaxChunk = 64;
constexpr int kCprPassRows = 8;  // state rows per workgroup of the pass

// The top tree level: this lane's half plus its partner's (lane ^ 1); both
// lanes get the same bits (IEEE addition is commutative).
__device__ __forceinline__ float pair_join(float x) { return x + dpp_mov<0xB1>(x); }

// bf16 element e (0..7) of a 16-byte LDS chunk, widened.
__device__ __forceinline__ float bf16_of(const u32x4 &w, int e)
{
    return (e & 1) ? __uint_as_float(w[e >> 1] & 0xffff0000u) : __uint_as_float(w[e >> 1] << 16);
}

// Balanced binary tree, in index order, over x[j] * y[j] for j < 64, with y a
// bf16 row in LDS read 16 bytes at a time.  The tree is kept as a binary
// counter: the trailing ones of j are the saved left siblings that product j
// closes, so the additions and their operand order are those of the
// level-by-level tree.
__device__ __forceinline__ float dot64(const float (&x)[64], const uint16_t *y)
{
    float st[6];
    float root = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const u32x4 w = reinterpret_cast<const u32x4 *>(y)[c];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = 8 * c + e;
            float t = x[j] * bf16_of(w, e);
            const int ones = __builtin_ctz(~static_cast<unsigned>(j));
            for (int l = 0; l < ones; ++l)
                t = st[l] + t;
            if (ones < 6)
                st[ones] = t;
            else
                root = t;
        }
    }
    return root;
}

// One token step on this lane's half row S (columns 64 hf .. 64 hf + 63 of
// row a).  k_row, q_row: the token's k and q rows in LDS; returns o[a].
__device__ __forceinline__ float cpr_token_step(float (&S)[64], const uint16_t *k_row,
                                                const uint16_t *q_row, float v_a, float alpha,
                                                float beta, int hf)
{
    const uint16_t *kh = k_row + 64 * hf;
    const float u = pair_join(dot64(S, kh));
    const float w = beta * (v_a - alpha * u);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const u32x4 kw = reinterpret_cast<const u32x4 *>(kh)[c];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            S[8 * c + e] = alpha * S[8 * c + e] + w * bf16_of(kw, e);
    }
    return pair_join(dot64(S, q_row + 64 * hf));
}

// Stage n token rows (128 bf16 each) of head h from [T][H][128] into
// dst[n][128], 16 bytes per thread and step.
__device__ __forceinline__ void stage_rows(const uint16_t *src, int64_t t0, int n, int64_t H,
                                           int64_t h, uint16_t (*dst)[kCprD])
{
    for (int e = threadIdx.x; e < n * 16; e += kCprThreads) {
        const int tok = e >> 4, part = e & 15;
        const u32x4 w =
            *reinterpret_cast<const u32x4 *>(src + ((t0 + tok) * H + h) * kCprD + part * 8);
        *reinterpret_cast<u32x4 *>(&dst[tok][part * 8]) = w;
    }
}

// Outputs of chunk blockIdx.y of head blockIdx.x: token steps from its
// boundary state bounds[c] ([c][H][128][128]).  The last chunk may be partial
// (T not a multiple of C): its stepped state goes to run_out.
__global__ __launch_bounds__(kCprThreads) void cpr_output_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    const float *__restrict__ bounds, float *__restrict__ o, float *__restrict__ run_out, int64_t T,
    int64_t H, int C)
{
    __shared__ __attribute__((aligned(16))) uint16_t ks[kCprMaxChunk][kCprD];
    __shared__ __attribute__((aligned(16))) uint16_t qs[kCprMaxChunk][kCprD];
    __shared__ __attribute__((aligned(16))) uint16_t vs[kCprMaxChunk][kCprD];
    __shared__ float al[kCprMaxChunk], be[kCprMaxChunk];
    const int64_t h = blockIdx.x;
    const int64_t c = blockIdx.y;
    const int64_t t0 = c * C;
    const int n = static_cast<int>(T - t0 < C ? T - t0 : C);
    stage_rows(k, t0, n, H, h, ks);
    stage_rows(q, t0, n, H, h, qs);
    stage_rows(v, t0, n, H, h, vs);
    for (int e = threadIdx.x; e < n; e += kCprThreads) {
        al[e] = alpha[(t0 + e) * H + h];
        be[e] = beta[(t0 + e) * H + h];
    }
    __syncthreads();
    const int a = threadIdx.x >> 1, hf = threadIdx.x & 1;
    float S[64];
    const float *B = bounds + ((c * H + h) * kCprD + a) * kCprD + 64 * hf;
#pragma unroll
    for (int j = 0; j < 64; j += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(B + j);
        S[j] = x[0];
        S[j + 1] = x[1];
        S[j + 2] = x[2];
        S[j + 3] = x[3];
    }
    for (int i = 0; i < n; ++i) {
        const float va = bf16_to_f32(vs[i][a]);
        const float oa = cpr_token_step(S, ks[i], qs[i], va, al[i], be[i], hf);
        if (hf == 0)
            o[((t0 + i) * H + h) * kCprD + a] = oa;
    }
    if (n < C && run_out) {
        float *R = run_out + (h * kCprD + a) * kCprD + 64 * hf;
#pragma unroll
        for (int j = 0; j < 64; j += 4)
            *reinterpret_cast<f32x4 *>(R + j) = f32x4{S[j], S[j + 1], S[j + 2], S[j + 3]};
    }
}

// Chunk form (P, U) of chunk blockIdx.y of head blockIdx.x, its tokens
// starting at t_first + blockIdx.y * C.  Lane pair j holds column j of R and
// of U, rows 64 hf .. 64 hf + 63 each.
__global__ __launch_bounds__(kCprThreads) void cpr_transition_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta, float *__restrict__ P,
    float *__restrict__ U, int64_t t_first, int64_t H, int C)
{
    __shared__ __attribute__((aligned(16))) uint16_t ks[kCprMaxChunk][kCprD];
    __shared__ __attribute__((aligned(16))) uint16_t vs[kCprMaxChunk][kCprD];
    __shared__ float al[kCprMaxChunk], be[kCprMaxChunk];
    const int64_t h = blockIdx.x;
    const int64_t c = blockIdx.y;
    const int64_t t0 = t_first + c * C;
    stage_rows(k, t0, C, H, h, ks);
    stage_rows(v, t0, C, H, h, vs);
    for (int e = threadIdx.x; e < C; e += kCprThreads) {
        al[e] = alpha[(t0 + e) * H + h];
        be[e] = beta[(t0 + e) * H + h];
    }
    __syncthreads();
    const int j = threadIdx.x >> 1, hf = threadIdx.x & 1;
    float R[64], Uc[64];
#pragma unroll
    for (int mi = 0; mi < 64; ++mi) {
        R[mi] = (64 * hf + mi == j) ? 1.0f : 0.0f;
        Uc[mi] = 0.0f;
    }
    for (int i = C - 1; i >= 0; --i) {
        const uint16_t *kh = ks[i] + 64 * hf;
        const uint16_t *vh = vs[i] + 64 * hf;
        const float r = pair_join(dot64(R, kh));  // products R[m] k[m] = k[m] R[m]
        const float a_i = al[i], b_i = be[i];
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            const u32x4 vw = reinterpret_cast<const u32x4 *>(vh)[cc];
            const u32x4 kw = reinterpret_cast<const u32x4 *>(kh)[cc];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t = b_i * bf16_of(vw, e);
                Uc[8 * cc + e] = Uc[8 * cc + e] + t * r;
                const float sm = b_i * bf16_of(kw, e);
                R[8 * cc + e] = a_i * (R[8 * cc + e] - sm * r);
            }
        }
    }
    float *Pc = P + (c * H + h) * kCprD * kCprD + j;
    float *Ucp = U + (c * H + h) * kCprD * kCprD + j;
#pragma unroll
    for (int mi = 0; mi < 64; ++mi) {
        Pc[(64 * hf + mi) * kCprD] = R[mi];
        Ucp[(64 * hf + mi) * kCprD] = Uc[mi];
    }
}

// Boundary pass for head blockIdx.x, state rows 8 blockIdx.y .. +7:
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lds_addr_of(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)p;
}

template <class T>
__device__ __forceinline__ void lds_pin(T &v)
{
    asm volatile("" : "+v"(v));
}

template <int N>
__device__ __forceinline__ void lgkm_wait()
{
    static_assert(N >= 0 && N <= 15, "lgkmcnt field");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

constexpr int kBlk = 8;                // terms per pipelined block of the pass
constexpr int kCprPassThreads = 512;   // two waves per SIMD

// LDS reads of terms M and M + 1 of the pass for a lane's 1 x 2 outputs:
// B[row][m], B[row][m+1] (8 bytes, the same address for every lane of a
// wave) and P[m][2q .. 2q+1], P[m+1][2q .. 2q+1] (rows 512 bytes apart: one
// ds_read2st64_b64 with offsets in units of 512 bytes).  Offsets are
// immediates: the largest, 127 x 512 bytes and 126 x 4 bytes, fit the
// instruction fields.
template <int M>
__device__ __forceinline__ void pass_pair_issue(f32x2 &b, f32x4 &p, uint32_t pa, uint32_t ba)
{
    asm volatile("ds_read2st64_b64 %0, %1 offset0:%2 offset1:%3"
                 : "=v"(p)
                 : "v"(pa), "n"(M), "n"(M + 1));
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(b) : "v"(ba), "n"(4 * M));
}

template <int K>
__device__ __forceinline__ void pass_block_issue(f32x2 (&bq)[kBlk / 2], f32x4 (&pq)[kBlk / 2],
                                                 uint32_t pa, uint32_t ba)
{
    static_assert(kBlk == 8, "four pairs of terms");
    pass_pair_issue<K * kBlk + 0>(bq[0], pq[0], pa, ba);
    pass_pair_issue<K * kBlk + 2>(bq[1], pq[1], pa, ba);
    pass_pair_issue<K * kBlk + 4>(bq[2], pq[2], pa, ba);
    pass_pair_issue<K * kBlk + 6>(bq[3], pq[3], pa, ba);
}

// B_{c+1} = U_c + B_c P_c for c < nb, from B_0 = S0 (zeros when null).
// bounds (optional) receives B_0 .. B_nb; snap receives B_nb, and run too
// when given.  S0 may alias snap (rows are read before they are written,
// each by the workgroup that owns them).
//
// A workgroup of eight waves owns 8 rows of one head; wave s computes row s
// and lane q columns 2q, 2q + 1: two products per term m from one value of
// B_c (a broadcast read) and two of P_c (consecutive across the lanes).  Two
// waves per SIMD hide each other's LDS and dependency latency.  P and B are
// double-buffered in LDS, so one barrier per chunk separates the reads of
// chunk c from the writes for chunk c + 1; P_{c+1} is written to LDS and
// P_{c+2} and U_{c+1} are loaded into registers while chunk c is multiplied.
__global__ __launch_bounds__(kCprPassThreads) void cpr_pass_kernel(
    const float *__restrict__ P, const float *__restrict__ U, const float *S0, float *bounds,
    float *snap, float *run, int64_t H, int64_t nb)
{
    __shared__ __attribute__((aligned(16))) float Ps[2][kCprD][kCprD];  // 128 KiB
    __shared__ __attribute__((aligned(16))) float Bs[2][kCprPassRows][kCprD];
    static_assert(kCprPassRows == 8 && kCprPassThreads == 8 * 64, "one row per wave");
    const int tid = static_cast<int>(threadIdx.x);
    const int s = tid >> 6;
    const int q = tid & 63;
    const int64_t hs = static_cast<int64_t>(blockIdx.x) * kCprD * kCprD;  // head's state offset
    const int64_t at = hs + (static_cast<int64_t>(blockIdx.y) * kCprPassRows + s) * kCprD + 2 * q;
    const int64_t state = H * kCprD * kCprD;  // one [H][128][128] block
    constexpr int kPer = kCprD * kCprD / 4 / kCprPassThreads;  // float4 of P per thread: 8
    f32x2 b = f32x2{0.0f, 0.0f};
    if (S0)
        b = *reinterpret_cast<const f32x2 *>(S0 + at);
    *reinterpret_cast<f32x2 *>(&Bs[0][s][2 * q]) = b;
    if (bounds)
        *reinterpret_cast<f32x2 *>(bounds + at) = b;
    f32x4 pn[kPer];
    f32x2 un = f32x2{0.0f, 0.0f};
    if (nb > 0) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(P + hs);
#pragma unroll
        for (int e = 0; e < kPer; ++e)
            reinterpret_cast<f32x4 *>(&Ps[0][0][0])[e * kCprPassThreads + tid] =
                src[e * kCprPassThreads + tid];
        if (nb > 1) {
            const f32x4 *nx = reinterpret_cast<const f32x4 *>(P + state + hs);
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                pn[e] = nx[e * kCprPassThreads + tid];
        }
        un = *reinterpret_cast<const f32x2 *>(U + at);
    }
    __syncthreads();
    for (int64_t c = 0; c < nb; ++c) {
        const int cur = static_cast<int>(c & 1);
        // P_{c+1} into the other buffer (last read in chunk c - 1, before the
        // barrier), then the loads of P_{c+2} and U_{c+1}: all of it overlaps
        // this chunk's products.
        f32x2 un_next = un;
        if (c + 1 < nb) {
#pragma unroll
            for (int e = 0; e < kPer; ++e)
                reinterpret_cast<f32x4 *>(&Ps[cur ^ 1][0][0])[e * kCprPassThreads + tid] = pn[e];
            if (c + 2 < nb) {
                const f32x4 *nx = reinterpret_cast<const f32x4 *>(P + (c + 2) * state + hs);
#pragma unroll
                for (int e = 0; e < kPer; ++e)
                    pn[e] = nx[e * kCprPassThreads + tid];
            }
            un_next = *reinterpret_cast<const f32x2 *>(U + (c + 1) * state + at);
        }
        float st[2][7];
        float root[2];
        // Software-pipelined over blocks of 8 terms: the LDS reads of block
        // k + 1 are in flight while block k is multiplied.  Reads and waits
        // are inline assembly, so their order is the one written here.
        const uint32_t pa = lds_addr_of(&Ps[cur][0][2 * q]);
        const uint32_t ba = lds_addr_of(&Bs[cur][s][0]);
        f32x2 bq[2][kBlk / 2];
        f32x4 pq[2][kBlk / 2];
        pass_block_issue<0>(bq[0], pq[0], pa, ba);
        static_for<kCprD / kBlk>([&](auto Kc) {
            constexpr int K = decltype(Kc)::value;
            constexpr int cb = K & 1;
            if constexpr (K + 1 < kCprD / kBlk) {
                pass_block_issue<K + 1>(bq[cb ^ 1], pq[cb ^ 1], pa, ba);
                lgkm_wait<kBlk>();  // block K landed, block K + 1 may be in flight
            } else {
                lgkm_wait<0>();
            }
#pragma unroll
            for (int i = 0; i < kBlk / 2; ++i) {
                lds_pin(bq[cb][i]);
                lds_pin(pq[cb][i]);
            }
#pragma unroll
            for (int i = 0; i < kBlk; ++i) {
                const int m = K * kBlk + i;
                // binary counter over the 128 products: the trailing ones of
                // m are the saved left siblings this product closes
                const int ones = __builtin_ctz(~static_cast<unsigned>(m));
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    float x = bq[cb][i >> 1][i & 1] * pq[cb][i >> 1][2 * (i & 1) + cc];
                    for (int lvl = 0; lvl < ones; ++lvl)
                        x = st[cc][lvl] + x;
                    if (ones < 7)
                        st[cc][ones] = x;
                    else
                        root[cc] = x;
                }
            }
        });
        b = f32x2{un[0] + root[0], un[1] + root[1]};
        *reinterpret_cast<f32x2 *>(&Bs[cur ^ 1][s][2 * q]) = b;
        if (bounds)
            *reinterpret_cast<f32x2 *>(bounds + (c + 1) * state + at) = b;
        un = un_next;
        lds_barrier();  // the loads of P_{c+2} stay in flight
    }
    *reinterpret_cast<f32x2 *>(snap + at) = b;
    if (run)
        *reinterpret_cast<f32x2 *>(run + at) = b;
}

// One decode step of token `pos` for every head: the running state run
// [H][128][128] is stepped in place and o [H][128] written.
__global__ __launch_bounds__(kCprThreads) void cpr_decode_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta, int64_t pos,
    float *__restrict__ run, float *__restrict__ o, int64_t H)
{
    __shared__ __attribute__((aligned(16))) uint16_t ks[1][kCprD];
    __shared__ __attribute__((aligned(16))) uint16_t qs[1][kCprD];
    __shared__ __attribute__((aligned(16))) uint16_t vs[1][kCprD];
    const int64_t h = blockIdx.x;
    stage_rows(k, pos, 1, H, h, ks);
    stage_rows(q, pos, 1, H, h, qs);
    stage_rows(v, pos, 1, H, h, vs);
    __syncthreads();
    const int a = threadIdx.x >> 1, hf = threadIdx.x & 1;
    float *Srow = run + (h * kCprD + a) * kCprD + 64 * hf;
    float S[64];
#pragma unroll
    for (int j = 0; j < 64; j += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(Srow + j);
        S[j] = x[0];
        S[j + 1] = x[1];
        S[j + 2] = x[2];
        S[j + 3] = x[3];
    }
    const float oa = cpr_token_step(S, ks[0], qs[0], bf16_to_f32(vs[0][a]), alpha[pos * H + h],
                                    beta[pos * H + h], hf);
    if (hf == 0)
        o[h * kCprD + a] = oa;
#pragma unroll
    for (int j = 0; j < 64; j += 4)
        *reinterpret_cast<f32x4 *>(Srow + j) = f32x4{S[j], S[j + 1], S[j + 2], S[j + 3]};
}

hipError_t launch_cpr_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const float *alpha, const float *beta, const float *S0, float *o,
                              float *snap, float *run, int64_t T, int64_t H, int C, float *P,
                              float *U, float *bounds, hipStream_t stream)
{
    const int64_t nb = T / C;
    const int64_t nchunks = (T + C - 1) / C;
    if (nb > 0)
        hipLaunchKernelGGL(cpr_transition_kernel, dim3(static_cast<unsigned>(H), static_cast<unsigned>(nb)),
                           dim3(kCprThreads), 0, stream, k, v, alpha, beta, P, U, int64_t{0}, H, C);
    hipLaunchKernelGGL(cpr_pass_kernel, dim3(static_cast<unsigned>(H), kCprD / kCprPassRows),
                       dim3(kCprPassThreads), 0, stream, P, U, S0, bounds, snap,
                       (T % C == 0) ? run : nullptr, H, nb);
    if (nchunks > 0)
        hipLaunchKernelGGL(cpr_output_kernel, dim3(static_cast<unsigned>(H), static_cast<unsigned>(nchunks)),
                           dim3(kCprThreads), 0, stream, q, k, v, alpha, beta, bounds, o,
                           (T % C == 0) ? nullptr : run, T, H, C);
    return hipGetLastError();
}

hipError_t launch_cpr_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const float *alpha, const float *beta, int64_t pos, float *snap,
                             float *run, float *o, int64_t H, int C, float *P, float *U,
                             hipStream_t stream)
{
    hipLaunchKernelGGL(cpr_decode_kernel, dim3(static_cast<unsigned>(H)), dim3(kCprThreads), 0, stream,
                       q, k, v, alpha, beta, pos, run, o, H);
    if ((pos + 1) % C == 0) {
        hipLaunchKernelGGL(cpr_transition_kernel, dim3(static_cast<unsigned>(H), 1u), dim3(kCprThreads), 0,
                           stream, k, v, alpha, beta, P, U, pos - (C - 1), H, C);
        hipLaunchKernelGGL(cpr_pass_kernel, dim3(static_cast<unsigned>(H), kCprD / kCprPassRows),
                           dim3(kCprPassThreads), 0, stream, P, U, snap, static_cast<float *>(nullptr),
                           snap, run, H, int64_t{1});
    }
    return hipGetLastError();
}

}  // namespace iso
