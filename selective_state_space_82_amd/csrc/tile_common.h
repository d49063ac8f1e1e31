// tile_common.h — wavefront tile staging helpers shared by the prefill and gradient kernels.
#pragma once

#include "device_common.h"

namespace ssm {

template <typename T> struct Chunk;  // 16 bytes of a row or run
template <> struct Chunk<float> { static constexpr int kElems = 4; };
template <> struct Chunk<uint16_t> { static constexpr int kElems = 8; };

// Widen one 16-byte chunk into `E` floats at dst (LDS).
template <typename T>
__device__ __forceinline__ void put_chunk(float *dst, const uint4 &v);
template <>
__device__ __forceinline__ void put_chunk<float>(float *dst, const uint4 &v) {
    *reinterpret_cast<float4 *>(dst) =
        make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
template <>
__device__ __forceinline__ void put_chunk<uint16_t>(float *dst, const uint4 &v) {
    *reinterpret_cast<float4 *>(dst) = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
    *reinterpret_cast<float4 *>(dst + 4) = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
}

// Widen one 16-byte chunk into `E` floats in registers.
template <typename T>
__device__ __forceinline__ void chunk_to_regs(float *dst, const uint4 &v);
template <>
__device__ __forceinline__ void chunk_to_regs<float>(float *dst, const uint4 &v) {
    dst[0] = __uint_as_float(v.x); dst[1] = __uint_as_float(v.y);
    dst[2] = __uint_as_float(v.z); dst[3] = __uint_as_float(v.w);
}
template <>
__device__ __forceinline__ void chunk_to_regs<uint16_t>(float *dst, const uint4 &v) {
    dst[0] = bf16_lo(v.x); dst[1] = bf16_hi(v.x); dst[2] = bf16_lo(v.y); dst[3] = bf16_hi(v.y);
    dst[4] = bf16_lo(v.z); dst[5] = bf16_hi(v.z); dst[6] = bf16_lo(v.w); dst[7] = bf16_hi(v.w);
}

// Narrow `E` floats into one 16-byte chunk of the storage type (bf16: round to nearest even).
template <typename T>
__device__ __forceinline__ uint4 regs_to_chunk(const float *v);
template <>
__device__ __forceinline__ uint4 regs_to_chunk<float>(const float *v) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
}
template <>
__device__ __forceinline__ uint4 regs_to_chunk<uint16_t>(const float *v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)narrow<uint16_t>(v[2 * i]) | ((uint32_t)narrow<uint16_t>(v[2 * i + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Load one chunk (E consecutive elements of a row or run starting at element t) with bounds;
// elements at or past `t_end` read as 0.
template <typename T>
__device__ __forceinline__ uint4 get_chunk(const T *__restrict__ row, int64_t t, int64_t t_end, bool row_ok,
                                           bool vec) {
    constexpr int E = Chunk<T>::kElems;
    uint4 r = make_uint4(0u, 0u, 0u, 0u);
    if (!row_ok) return r;
    if (vec && t + E <= t_end) return *reinterpret_cast<const uint4 *>(row + t);
    T tmp[E];
#pragma unroll
    for (int e = 0; e < E; ++e) tmp[e] = (t + e < t_end) ? row[t + e] : T(0);
    __builtin_memcpy(&r, tmp, sizeof(r));
    return r;
}

// p[ok ? i : 0] with the load issued unconditionally (a guarded load would become a branch
// with a wait behind it), then `fallback` where !ok. p[0] must be readable.
__device__ __forceinline__ float load_or(const float *p, int64_t i, bool ok, float fallback) {
    const float v = p[ok ? i : 0];
    return ok ? v : fallback;
}

// U consecutive floats from LDS (U = 1, 2 or 4).
template <int U>
__device__ __forceinline__ void lds_get(const float *p, float (&o)[U]) {
    if constexpr (U == 4) {
        const float4 v = *reinterpret_cast<const float4 *>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else if constexpr (U == 2) {
        const float2 v = *reinterpret_cast<const float2 *>(p);
        o[0] = v.x; o[1] = v.y;
    } else {
        o[0] = *p;
    }
}

// Orders this wave's LDS accesses around a hand-off between its lanes (tile stores -> scan
// reads, partial sums -> transposed reads, outputs -> line stores). One wave's LDS operations
// execute in order, so this only fences the compiler; it emits no wait.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Value of `v` held by lane (lane ^ 1) or (lane ^ 2) of the same quad: DPP quad permutes.
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the G (1, 2 or 4) adjacent lanes of a quad: an xor butterfly of DPP quad permutes; every
// lane of the group ends with bitwise the same value (addition is commutative).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v += quad_perm<0xB1>(v);  // quad_perm [1, 0, 3, 2]
    if constexpr (G >= 4) v += quad_perm<0x4E>(v);  // quad_perm [2, 3, 0, 1]
    return v;
}

}  // namespace ssm
