// device_common.h — storage helpers shared by the prefill and decode kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kWave = 64;

// Storage types: fp32 is `float`, bf16 is its bit pattern in `uint16_t`.
__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float widen(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// bf16 pairs packed in a dword: element 0 in the low half, element 1 in the high half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T> __device__ __forceinline__ T narrow(float v);
template <> __device__ __forceinline__ float narrow<float>(float v) { return v; }
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ uint16_t narrow<uint16_t>(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// v_exp_f32: 2^v, about 1 ulp; flushes to 0 far below the normal range.
__device__ __forceinline__ float exp2_fast(float v) { return __builtin_amdgcn_exp2f(v); }

// silu(v) = v / (1 + e^{-v}), with the hardware exp and reciprocal.
__device__ __forceinline__ float silu(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + exp2_fast(-kLog2e * v));
}

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^{−|v|}), with log1p from its series e − e²/2 + e³/3
// where e < 2^-5 (relative error below 8e-6; 1 + e would round away most of e there) and from the hardware
// log of 1 + e elsewhere.
__device__ __forceinline__ float softplus(float v) {
    const float e = exp2_fast(-kLog2e * __builtin_fabsf(v));
    const float series = e * __builtin_fmaf(e, __builtin_fmaf(e, 1.0f / 3.0f, -0.5f), 1.0f);
    const float direct = __builtin_amdgcn_logf(1.0f + e) * 0.69314718055994530942f;
    return __builtin_fmaxf(v, 0.0f) + (e < 0.03125f ? series : direct);
}

// (e^{v} - 1) / v for |v| < 2^-4 by its Taylor series (relative error below 1e-8 there).
__device__ __forceinline__ float expm1_over_v_small(float v) {
    return __builtin_fmaf(v, __builtin_fmaf(v, __builtin_fmaf(v, 1.0f / 24.0f, 1.0f / 6.0f), 0.5f), 1.0f);
}

// e^v − 1 from u = v·log2(e) and abar = 2^u: the series near v = 0 (no cancellation), else abar − 1.
__device__ __forceinline__ float expm1_log2(float u, float abar) {
    const float v = u * 0.69314718055994530942f;
    return __builtin_fabsf(v) < 0.0625f ? v * expm1_over_v_small(v) : abar - 1.0f;
}

// ZOH input coefficient (e^{Δa} − 1)/a for one state, given abar = e^{Δa} and inv_a = 1/a.
// Near Δa = 0 the quotient is taken from its series, so a = 0 yields the limit Δ exactly and
// tiny |a| does not cancel.
__device__ __forceinline__ float zoh_input_coef(float dt, float a, float abar, float inv_a) {
    const float v = dt * a;
    const float near0 = dt * expm1_over_v_small(v);
    const float far = (abar - 1.0f) * inv_a;  // NaN at a = 0, never selected there
    return __builtin_fabsf(v) < 0.0625f ? near0 : far;
}

// The same coefficient from u = Δ·a·log2(e) (the argument already formed for exp2), so the
// caller need not keep a itself: v = u·ln 2.
__device__ __forceinline__ float zoh_input_coef_log2(float dt, float u, float abar, float inv_a) {
    const float v = u * 0.69314718055994530942f;
    const float near0 = dt * expm1_over_v_small(v);
    const float far = (abar - 1.0f) * inv_a;  // NaN at a = 0, never selected there
    return __builtin_fabsf(v) < 0.0625f ? near0 : far;
}

}  // namespace ssm
