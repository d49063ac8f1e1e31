// ssd_common.h — what the two translation units of the scalar-decay chunked form share: the chunk
// geometry, the kernel arguments, the MFMA tile helpers and the launcher of the fused state walk.
// The fused walk has a translation unit of its own (ssd_scan.hip) so that its LDS layout does not
// change how the compiler lays out and addresses the other kernels' LDS.
#pragma once

#include "device_common.h"

namespace ssm {
namespace ssd {

typedef float f16v __attribute__((ext_vector_type(16)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

constexpr int kQ = 64;           // chunk length
constexpr int kP = 64;           // channels per head
constexpr int kThreads = 256;    // four wavefronts
constexpr int kMS = kQ + 4;      // LDS row stride (fp32) of 64-step rows (16-byte aligned rows)
constexpr int kMH = kQ + 8;      // LDS row stride (bf16 elements) of 64-step rows: 144 bytes, 16-byte aligned

struct SsdArgs {
    const void *x, *delta, *B, *C, *z;
    const float *A, *D, *h0;
    void *y;
    float *hT;
    float *S;      // [b][H][nc][P][N] chunk states, then entering states
    float *decay;  // [b][H][nc]
    int64_t b, H, L, nc;
    bool vec;      // x, z and y rows allow 16-byte (fp32) / 8-byte (bf16) accesses at 4-element steps
    bool vec_bc;   // so do the rows of B and C
    bool vec8;     // x rows allow 16-byte loads at 8-element steps (bf16)
    bool fused;    // chunk states and their pass in one kernel (ssd_scan_kernel)
    bool vec_bc16; // B and C allow 16-byte loads (bf16 rows of N >= 64)
    bool fused_all;// the whole chunked form in one ordered walk per (b, head) (ssd_fused_kernel)
};

__device__ __forceinline__ int lane() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave() { return threadIdx.x >> 6; }

// Row position of result register r of lane l in a 32×32 tile.
__device__ __forceinline__ int d_row(int r, int l) { return 8 * (r / 4) + 4 * (l / 32) + (r % 4); }

// Four consecutive elements row[i .. i+3] as fp32, zeros at and past `limit`; one 16-byte (fp32) or
// 8-byte (bf16) load when `vec` says the row allows it.
template <typename T>
__device__ __forceinline__ float4 load4(const T *row, int64_t i, int64_t limit, bool vec) {
    if (vec && i + 4 <= limit) {
        if constexpr (sizeof(T) == 4) {
            return *reinterpret_cast<const float4 *>(row + i);
        } else {
            const uint2 w = *reinterpret_cast<const uint2 *>(row + i);
            return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
        }
    }
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = i + e < limit ? widen(row[i + e]) : 0.0f;
    return make_float4(v[0], v[1], v[2], v[3]);
}

// One 32×32 tile product over K = 2W with the K index permuted so that each lane reads a contiguous run:
// at step j the lower lane half supplies k = j and the upper half k = W + j. fa(j) / fb(j) return the
// lane's operand values for steps j .. j+3 (its own row, k = hi·W + j .. +3).
// All operand loads are issued before the first product (fully unrolled), so their latencies overlap.
template <int W, typename FA, typename FB>
__device__ __forceinline__ void mfma_tile(f16v &acc, FA fa, FB fb) {
    float4 a4[W / 4], b4[W / 4];
#pragma unroll
    for (int j = 0; j < W / 4; ++j) {
        a4[j] = fa(4 * j);
        b4[j] = fb(4 * j);
    }
#pragma unroll
    for (int j = 0; j < W / 4; ++j) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[j].x, b4[j].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[j].y, b4[j].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[j].z, b4[j].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[j].w, b4[j].w, acc, 0, 0, 0);
    }
}

// Eight fp32 values as bf16 hi = bf16(v) and lo = bf16(v − hi).
__device__ __forceinline__ void split8(const float4 &u, const float4 &v, bf8v &hi8, bf8v &lo8) {
    const float f[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 hb = (__bf16)f[e];
        hi8[e] = hb;
        lo8[e] = (__bf16)(f[e] - (float)hb);
    }
}

// One 32×32 tile product over K = 2W on the bf16 MFMA, K split across the lane halves as in mfma_tile:
// at step j the lower half supplies k = 8j .. 8j+7 and the upper half k = W + 8j .. +7, so each lane
// reads 16 contiguous bytes of its own LDS row per step.
template <int W>
__device__ __forceinline__ void mfma_tile_bf16(f16v &acc, const uint16_t *arow, const uint16_t *brow) {
    bf8v a8[W / 8], b8[W / 8];
#pragma unroll
    for (int j = 0; j < W / 8; ++j) {
        a8[j] = *reinterpret_cast<const bf8v *>(arow + 8 * j);
        b8[j] = *reinterpret_cast<const bf8v *>(brow + 8 * j);
    }
#pragma unroll
    for (int j = 0; j < W / 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8[j], b8[j], acc, 0, 0, 0);
}

// As mfma_tile_bf16 with one operand an fp32 LDS row entering as hi + lo (two products per step);
// SPLIT_A says which operand is the fp32 one.
template <int W, bool SPLIT_A>
__device__ __forceinline__ void mfma_tile_split(f16v &acc, const float *frow, const uint16_t *brow) {
#pragma unroll
    for (int j = 0; j < W / 8; ++j) {
        bf8v h8, l8;
        split8(*reinterpret_cast<const float4 *>(frow + 8 * j), *reinterpret_cast<const float4 *>(frow + 8 * j + 4),
               h8, l8);
        const bf8v o8 = *reinterpret_cast<const bf8v *>(brow + 8 * j);
        if (SPLIT_A) {
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h8, o8, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l8, o8, acc, 0, 0, 0);
        } else {
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o8, h8, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o8, l8, acc, 0, 0, 0);
        }
    }
}

// The whole chunked form for bf16 storage in one ordered walk per (b, head) (ssd_scan.hip); N is 64 or 128.
hipError_t launch_fused(const SsdArgs &a, int64_t N, hipStream_t stream);

// The chunk states' walk of ssd_scan.hip (one launch): the state entering every chunk into a.S and the
// final state into a.hT. N is 64 or 128.
hipError_t launch_state_walk(const SsdArgs &a, int64_t N, bool bf16, hipStream_t stream);

}  // namespace ssd
}  // namespace ssm
