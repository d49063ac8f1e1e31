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
#include "device_common.h"
#include "launch.h"

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
    int vec;  // N % 4 == 0 and 16-byte aligned state/A rows
};

template <typename T, int LP>
__global__ __launch_bounds__(256) void scan_step_kernel(StepArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t pair = gid / LP;
    const int q = (int)(gid % LP);
    if (pair >= a.b * a.d) return;  // whole LP groups leave together: the grid ends on a group edge
    const int64_t bi = pair / a.d;
    const int64_t ch = pair - bi * a.d;
    const int n0 = q * 4;
    const int nvalid = (int)((a.N - n0) < 4 ? (a.N - n0) : 4);

    const T *__restrict__ xg = static_cast<const T *>(a.x);
    const T *__restrict__ dg = static_cast<const T *>(a.delta);
    const T *__restrict__ zg = static_cast<const T *>(a.z);
    const T *__restrict__ Bg = static_cast<const T *>(a.B) + bi * a.N;
    const T *__restrict__ Cg = static_cast<const T *>(a.C) + bi * a.N;

    const float xt = widen(xg[pair]);
    const float dt = widen(dg[pair]);
    float h[4] = {0.f, 0.f, 0.f, 0.f}, Av[4] = {-1.f, -1.f, -1.f, -1.f};
    float Bv[4] = {0.f, 0.f, 0.f, 0.f}, Cv[4] = {0.f, 0.f, 0.f, 0.f};
    float *st = a.state + pair * a.N + n0;
    const float *Ar = a.A + ch * a.N + n0;
    if (a.vec && nvalid == 4) {
        const float4 hv = *reinterpret_cast<const float4 *>(st);
        const float4 av = *reinterpret_cast<const float4 *>(Ar);
        h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
        Av[0] = av.x; Av[1] = av.y; Av[2] = av.z; Av[3] = av.w;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j < nvalid) { h[j] = st[j]; Av[j] = Ar[j]; }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (j < nvalid) { Bv[j] = widen(Bg[n0 + j]); Cv[j] = widen(Cg[n0 + j]); }

    float acc = 0.0f;
    const float bx_scale = xt;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float abar = exp2_fast(dt * (Av[j] * kLog2e));
        const float kc = zoh_input_coef(dt, Av[j], abar, 1.0f / Av[j]);
        h[j] = __builtin_fmaf(abar, h[j], kc * (Bv[j] * bx_scale));
        acc = __builtin_fmaf(Cv[j], h[j], acc);
    }
#pragma unroll
    for (int m = 1; m < LP; m <<= 1) acc += __shfl_xor(acc, m, LP);

    if (a.vec && nvalid == 4) {
        *reinterpret_cast<float4 *>(st) = make_float4(h[0], h[1], h[2], h[3]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j < nvalid) st[j] = h[j];
    }
    if (q == 0) {
        float v = acc;
        if (a.D) v = __builtin_fmaf(a.D[ch], xt, v);
        if (zg) v *= silu(widen(zg[pair]));
        static_cast<T *>(a.y)[pair] = narrow<T>(v);
    }
}

template <typename T>
hipError_t launch_step_typed(const StepArgs &a, hipStream_t stream) {
    const int lp_needed = (int)((a.N + 3) / 4);
    int lp = 1;
    while (lp < lp_needed) lp <<= 1;
    const int64_t threads = a.b * a.d * lp;
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    switch (lp) {
        case 1: hipLaunchKernelGGL((scan_step_kernel<T, 1>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((scan_step_kernel<T, 2>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((scan_step_kernel<T, 4>), grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL((scan_step_kernel<T, 8>), grid, block, 0, stream, a); break;
        case 16: hipLaunchKernelGGL((scan_step_kernel<T, 16>), grid, block, 0, stream, a); break;
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
    if (p.bf16) return launch_step_typed<uint16_t>(a, stream);
    return launch_step_typed<float>(a, stream);
}

}  // namespace ssm
