// scan_step.hip — decode: one recurrent step of the selective scan on a state kept in HBM.
//
// Method (page "Mambaとは？Transformer以外の系列モデル", section training、prefill、decodeでは計算の
// 姿が違う: each new token updates every layer's SSM state once; page "State Space Models（SSM）と
// Mamba" §2.4 and §5.1: recurrent mode, O(d·N) per token with a fixed-size state).
//
// The step is bound by HBM traffic (the fp32 state is read and written once per token), so the
// layout serves coalescing: `LP` consecutive lanes share one (b, d) row, each owning 4 consecutive
// states, so a wavefront reads and writes one contiguous run of 64 × 16 bytes of state. The
// readout partials of the LP lanes are combined by an xor butterfly (identical sum on every lane),
// and the first lane of the row applies the skip term and gate and stores y.
//
// The CONV variant is the whole decode step of the Mamba block's main branch (page "Mambaとは？Transformer
// 以外の系列モデル", section training、prefill、decodeでは計算の姿が違う: each layer keeps a Conv1D state and
// an SSM state): the token's raw input goes through the causal Conv1D against the stored last W − 1
// inputs, plus bias and SiLU, and Δ gets its bias (and softplus); the Conv1D state shifts by one in the
// same launch.
#include "device_common.h"
#include "launch.h"

#ifndef SSM_STEP_R
#define SSM_STEP_R 2  // pairs per lane group (loads in flight per lane)
#endif

namespace ssm {
namespace {

struct StepArgs {
    float *state;
    const void *x, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z;
    void *y;
    int64_t b, d, N;
    int vec;     // N % 4 == 0 and 16-byte aligned state/A rows
    int vec_bc;  // N % 4 == 0 and B/C rows aligned to 4 elements
    // CONV: x is the raw input; conv_state [b][d][conv_W − 1] fp32, shifted in place
    float *conv_state;
    const float *conv_w, *conv_bias, *delta_bias;
    void *x_out;
    int conv_W, delta_softplus;
};

// Four consecutive B or C values (one lane's states) in one load when aligned.
template <typename T>
__device__ __forceinline__ void load4(const T *p, float (&o)[4]);
template <>
__device__ __forceinline__ void load4<float>(const float *p, float (&o)[4]) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t *p, float (&o)[4]) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
}

typedef float f4v __attribute__((ext_vector_type(4)));

// LP lanes per (b, d) pair, R pairs per lane group: a block of 256 threads covers R * 256 / LP
// consecutive pairs, and every lane issues the loads of its R pairs before any arithmetic, so
// R state reads per lane are in flight at once. The state streams through (read once, written
// once) with non-temporal accesses.
template <typename T, int LP, int R, bool CONV = false>
__global__ __launch_bounds__(256) void scan_step_kernel(StepArgs a) {
    constexpr int PB = 256 / LP;  // pairs per block and round
    const uint32_t bd = (uint32_t)(a.b * a.d);
    const uint32_t d = (uint32_t)a.d;
    const int q = threadIdx.x % LP;
    const int n0 = q * 4;
    const int nvalid = (int)((a.N - n0) < 4 ? (a.N - n0) : 4);
    const bool full = a.vec && nvalid == 4;
    const bool full_bc = a.vec_bc && nvalid == 4;

    const T *__restrict__ xg = static_cast<const T *>(a.x);
    const T *__restrict__ dg = static_cast<const T *>(a.delta);
    const T *__restrict__ zg = static_cast<const T *>(a.z);

    uint32_t pair[R];
    bool ok[R];
    float xt[R], dt[R], zt[R], dsk[R];
    float raw[R], cs[R][3];  // CONV: the raw input and the stored inputs before it (oldest first)
    float h[R][4], Av[R][4], Bv[R][4], Cv[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t pr = (uint32_t)blockIdx.x * (R * PB) + r * PB + threadIdx.x / LP;
        ok[r] = pr < bd;
        pair[r] = ok[r] ? pr : 0u;  // lanes past the end read pair 0 and store nothing
        const uint32_t bi = pair[r] / d;
        const uint32_t ch = pair[r] - bi * d;
        xt[r] = widen(xg[pair[r]]);
        dt[r] = widen(dg[pair[r]]);
        if constexpr (CONV) {
            const int H = a.conv_W - 1;
            const float *st = a.conv_state + (int64_t)pair[r] * H;
            const float *w = a.conv_w + (int64_t)ch * a.conv_W;
            raw[r] = xt[r];
            float u = a.conv_bias ? a.conv_bias[ch] : 0.0f;
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                cs[r][k] = k < H ? st[k] : 0.0f;
                if (k < H) u = __builtin_fmaf(w[k], cs[r][k], u);
            }
            u = __builtin_fmaf(w[H], raw[r], u);
            xt[r] = silu(u);
            float v = dt[r] + (a.delta_bias ? a.delta_bias[ch] : 0.0f);
            dt[r] = a.delta_softplus ? softplus(v) : v;
        }
        zt[r] = zg ? widen(zg[pair[r]]) : 0.0f;
        dsk[r] = a.D ? a.D[ch] : 0.0f;
        const float *st = a.state + (int64_t)pair[r] * a.N + n0;
        const float *Ar = a.A + (int64_t)ch * a.N + n0;
        const T *Bg = static_cast<const T *>(a.B) + (int64_t)bi * a.N + n0;
        const T *Cg = static_cast<const T *>(a.C) + (int64_t)bi * a.N + n0;
        if (full) {
            const f4v hv = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(st));
            const float4 av = *reinterpret_cast<const float4 *>(Ar);
            h[r][0] = hv.x; h[r][1] = hv.y; h[r][2] = hv.z; h[r][3] = hv.w;
            Av[r][0] = av.x; Av[r][1] = av.y; Av[r][2] = av.z; Av[r][3] = av.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h[r][j] = j < nvalid ? st[j] : 0.0f;
                Av[r][j] = j < nvalid ? Ar[j] : -1.0f;
            }
        }
        if (full_bc) {
            load4<T>(Bg, Bv[r]);
            load4<T>(Cg, Cv[r]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                Bv[r][j] = j < nvalid ? widen(Bg[j]) : 0.0f;
                Cv[r][j] = j < nvalid ? widen(Cg[j]) : 0.0f;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float abar = exp2_fast(dt[r] * (Av[r][j] * kLog2e));
            const float kc = zoh_input_coef(dt[r], Av[r][j], abar, 1.0f / Av[r][j]);
            h[r][j] = __builtin_fmaf(abar, h[r][j], kc * (Bv[r][j] * xt[r]));
            acc = __builtin_fmaf(Cv[r][j], h[r][j], acc);
        }
#pragma unroll
        for (int m = 1; m < LP; m <<= 1) acc += __shfl_xor(acc, m, LP);
        if (!ok[r]) continue;
        float *st = a.state + (int64_t)pair[r] * a.N + n0;
        if (full) {
            f4v hw;
            hw.x = h[r][0]; hw.y = h[r][1]; hw.z = h[r][2]; hw.w = h[r][3];
            __builtin_nontemporal_store(hw, reinterpret_cast<f4v *>(st));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j < nvalid) st[j] = h[r][j];
        }
        if (q == 0) {
            float v = __builtin_fmaf(dsk[r], xt[r], acc);
            if (zg) v *= silu(zt[r]);
            static_cast<T *>(a.y)[pair[r]] = narrow<T>(v);
            if constexpr (CONV) {  // the Conv1D state moves on by one input; the convolved input goes out
                const int H = a.conv_W - 1;
                float *st = a.conv_state + (int64_t)pair[r] * H;
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    if (k < H) st[k] = k + 1 < H ? cs[r][k + 1] : raw[r];
                if (a.x_out) static_cast<T *>(a.x_out)[pair[r]] = narrow<T>(xt[r]);
            }
        }
    }
}

template <typename T, bool CONV>
hipError_t launch_step_typed(const StepArgs &a, hipStream_t stream) {
    const int lp_needed = (int)((a.N + 3) / 4);
    int lp = 1;
    while (lp < lp_needed) lp <<= 1;
    constexpr int R = SSM_STEP_R;
    const int64_t per_block = (int64_t)R * (256 / lp);
    const dim3 grid((unsigned)((a.b * a.d + per_block - 1) / per_block)), block(256);
    switch (lp) {
        case 1: hipLaunchKernelGGL((scan_step_kernel<T, 1, R, CONV>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((scan_step_kernel<T, 2, R, CONV>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((scan_step_kernel<T, 4, R, CONV>), grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL((scan_step_kernel<T, 8, R, CONV>), grid, block, 0, stream, a); break;
        case 16: hipLaunchKernelGGL((scan_step_kernel<T, 16, R, CONV>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_step(const StepLaunch &p, hipStream_t stream) {
    StepArgs a{};
    a.state = p.state; a.x = p.x; a.delta = p.delta; a.A = p.A; a.B = p.B; a.C = p.C; a.D = p.D;
    a.z = p.z; a.y = p.y; a.b = p.b; a.d = p.d; a.N = p.N;
    auto al16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
    a.vec = (p.N % 4 == 0) && al16(p.state) && al16(p.A);
    const uintptr_t bc_align = p.bf16 ? 8u : 16u;
    a.vec_bc = (p.N % 4 == 0) && (reinterpret_cast<uintptr_t>(p.B) % bc_align == 0) &&
               (reinterpret_cast<uintptr_t>(p.C) % bc_align == 0);
    a.conv_state = p.conv_state; a.conv_w = p.conv_w; a.conv_bias = p.conv_bias; a.delta_bias = p.delta_bias;
    a.x_out = p.x_out; a.conv_W = p.conv_W; a.delta_softplus = p.delta_softplus;
    if (p.conv_w) return p.bf16 ? launch_step_typed<uint16_t, true>(a, stream) : launch_step_typed<float, true>(a, stream);
    if (p.bf16) return launch_step_typed<uint16_t, false>(a, stream);
    return launch_step_typed<float, false>(a, stream);
}

}  // namespace ssm
