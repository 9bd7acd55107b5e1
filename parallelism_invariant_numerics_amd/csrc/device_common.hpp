// device_common.hpp -- shared device helpers for the gfx950 kernels.
//
// Every kernel that produces or consumes the invariant numbers uses these
// single definitions (bf16 rounding, exp/log, the fixed-tree folds), compiled
// with the same flags (no fast-math, no FP contraction), so the same inputs
// give the same bits in every kernel that calls them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace iso {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
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


// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b)
{
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bit pattern, round to nearest, ties to even (finite inputs;
// infinities stay infinite, NaN stays NaN).  Written as a select rather than
// a branch, so that kernels converting many values in a row keep straight-
// line code.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    // 0x40 (a quiet-NaN bit) when the low half is nonzero, without a compare
    const uint32_t special = (u >> 16) | ((((u & 0xffffu) + 0xffffu) >> 16) << 6);
    return static_cast<uint16_t>((u & 0x7f800000u) == 0x7f800000u ? special : rounded);
}

// e^x for x <= 0 as 2^(x * log2 e) on the hardware exp2 (one rounding of the
// product, then v_exp_f32).  Used for every softmax term in the library.
__device__ __forceinline__ float exp_neg(float x)
{
    const float kLog2e = 1.44269504088896340736f;
    return __builtin_amdgcn_exp2f(x * kLog2e);
}

// SwiGLU activation of one element, silu(g) * u with silu(g) = g / (1 + e^-g)
// (e^-g on the hardware exp2, as in exp_neg); FP32, no contraction.  The MoE
// gate/up epilogue and iso_swiglu share it, so the same (g, u) bits give the
// same activation bits in both.
__device__ __forceinline__ float swiglu_act(float g, float u)
{
    const float kLog2e = 1.44269504088896340736f;
    const float ex = __builtin_amdgcn_exp2f(-g * kLog2e);
    return (g / (1.0f + ex)) * u;
}

// Natural log for the final logprob (one call per row): ROCm's logf.
__device__ __forceinline__ float log_f32(float x) { return logf(x); }

// The softmax chunk merge (m, s) + (m', s') = (u, s e^(m-u) + s' e^(m'-u)),
// u = max(m, m').  Commutative bit for bit; (-inf, 0) is its identity, and
// two identities give the identity (never exp(-inf - -inf)).
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2)
{
    float u = fmaxf(m, m2);
    if (u == -INFINITY) {
        m = -INFINITY;
        s = 0.0f;
        return;
    }
    float a = s * exp_neg(m - u);
    float b = s2 * exp_neg(m2 - u);
    m = u;
    s = a + b;
}

// Butterfly exchange within a wave (lane ^ mask), via ds_swizzle/bpermute.
__device__ __forceinline__ float shfl_xor(float v, int mask)
{
    return __shfl_xor(v, mask, kWave);
}

// Butterflies over the 16 lanes of a DPP row with the partners (l, l^1),
// (l, l^2), (l, l^4), (l, l^8), on DPP moves instead of LDS permutes.  The
// first two steps use exact xor patterns (quad_perm [1,0,3,2], [2,3,0,1]);
// after them every quad holds one value, so the 8-lane half mirror and the
// 16-lane mirror read the same partner values as xor 4 and xor 8.  Every
// lane ends with the same result, and a sum is the balanced tree over the 16
// lanes in index order (IEEE addition is commutative, so a + b in one lane
// and b + a in its partner agree).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float row16_sum(float e)
{
    e = e + dpp_mov<0xB1>(e);   // quad_perm [1,0,3,2]: l ^ 1
    e = e + dpp_mov<0x4E>(e);   // quad_perm [2,3,0,1]: l ^ 2
    e = e + dpp_mov<0x141>(e);  // row_half_mirror: the other quad of the 8
    e = e + dpp_mov<0x140>(e);  // row_mirror: the other 8 of the 16
    return e;
}
__device__ __forceinline__ float row16_max(float m)
{
    m = fmaxf(m, dpp_mov<0xB1>(m));
    m = fmaxf(m, dpp_mov<0x4E>(m));
    m = fmaxf(m, dpp_mov<0x141>(m));
    m = fmaxf(m, dpp_mov<0x140>(m));
    return m;
}

// Workgroup barrier for code that has global loads in flight which the
// barrier must not wait for (__syncthreads() may also drain the vector
// memory counter): LDS operations complete first, then all waves meet.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace iso
