// conv1d.hip — the short causal depthwise Conv1D (+ SiLU) that feeds the scan in a Mamba block, and
// its decode step.
//
// Page "Mambaとは？Transformer以外の系列モデル": section Mamba blockのarchitecture (the main branch mixes
// neighbouring tokens with a short causal Conv1D, applies SiLU, then the selective SSM) and section
// training、prefill、decodeでは計算の姿が違う (in decode each layer keeps a Conv1D state next to its SSM
// state). Per channel d with taps w[d][0..W) and bias c_d:
//   u_t = c_d + Σ_{k<W} w[d][k] · xin_{t−(W−1)+k},   x_t = silu(u_t)  (or u_t),
// inputs before t = 0 coming from the state (the W − 1 preceding inputs, oldest first) or zero.
//
// Bound by HBM traffic. A workgroup of 256 threads covers 256 consecutive 16-byte chunks of one (b, d)
// row, so the row, the channel, its taps and bias are workgroup-uniform (scalar registers); each thread
// produces one chunk (4 fp32 or 8 bf16 outputs) from that chunk of the input and the W − 1 inputs before
// it (the previous chunk, read again by the neighbouring lane through the caches). The output streams out
// with non-temporal stores (written once, read by a later kernel). Measured on the 1.4B-like shape: more
// chunks per thread, or larger workgroups, ran slower; non-temporal loads too.
#include "device_common.h"
#include "launch.h"
#include "tile_common.h"

namespace ssm {
namespace {

constexpr int kConvBlock = 256;

struct ConvArgs {
    const void *xin;
    const float *w, *bias, *state_in;
    void *xout;
    float *state_out;
    int64_t b, d, L;
    int64_t tiles_per_row, n_blocks;
    int silu_on;
    int vec;         // rows allow 16-byte accesses
    int fuse_state;  // the conv kernel writes state_out itself (no aliasing, L >= W - 1)
};

typedef unsigned u4v __attribute__((ext_vector_type(4)));

template <typename T, int W>
__global__ __launch_bounds__(kConvBlock) void conv1d_kernel(ConvArgs a) {
    constexpr int E = Chunk<T>::kElems;
    constexpr int H = W - 1;
    constexpr int P = (H + E - 1) / E;  // previous chunks needed (0 or 1 for W <= E + 1)
    for (int64_t blk = blockIdx.x; blk < a.n_blocks; blk += gridDim.x) {
        const int64_t row = blk / a.tiles_per_row;  // uniform across the workgroup
        const int64_t tile = blk - row * a.tiles_per_row;
        const int64_t ch = row % a.d;
        const T *xr = static_cast<const T *>(a.xin) + row * a.L;
        T *yr = static_cast<T *>(a.xout) + row * a.L;
        const int64_t t0 = (tile * kConvBlock + threadIdx.x) * E;
        if (t0 >= a.L) continue;

        // ext[0 .. P*E) = inputs t0 − P*E .. t0 − 1 (from the row, or the state before t = 0);
        // ext[P*E ..) = the chunk itself
        float ext[(P + 1) * E];
        const bool full = a.vec && t0 + E <= a.L;
        if (full) {
            chunk_to_regs<T>(ext + P * E, *reinterpret_cast<const uint4 *>(xr + t0));
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) ext[P * E + e] = (t0 + e < a.L) ? widen(xr[t0 + e]) : 0.0f;
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int64_t tp = t0 - (P - p) * E;  // first step of this previous chunk
            if (tp >= 0 && a.vec) {
                chunk_to_regs<T>(ext + p * E, *reinterpret_cast<const uint4 *>(xr + tp));
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int64_t t = tp + e;
                    float v = 0.0f;
                    if (t >= 0) v = widen(xr[t]);
                    else if (a.state_in && t >= -H) v = a.state_in[row * H + (H + t)];
                    ext[p * E + e] = v;
                }
            }
        }
        float wk[W];
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k] = a.w[ch * W + k];
        const float c = a.bias ? a.bias[ch] : 0.0f;
        float out[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float u = c;
#pragma unroll
            for (int k = 0; k < W; ++k) u = __builtin_fmaf(wk[k], ext[P * E + e - H + k], u);
            out[e] = a.silu_on ? silu(u) : u;
        }
        if (full) {
            T packed[E];
#pragma unroll
            for (int e = 0; e < E; ++e) packed[e] = narrow<T>(out[e]);
            u4v v;
            __builtin_memcpy(&v, packed, sizeof(v));
            __builtin_nontemporal_store(v, reinterpret_cast<u4v *>(yr + t0));
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (t0 + e < a.L) yr[t0 + e] = narrow<T>(out[e]);
        }
        if (H > 0 && a.fuse_state && t0 + E > a.L - H) {
            // this chunk holds some of the last W − 1 inputs, which become the state
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int64_t k = t0 + e - (a.L - H);
                if (k >= 0 && k < H) a.state_out[row * H + k] = ext[P * E + e];
            }
        }
    }
}

// The state left behind: the last W − 1 inputs of (state_in, xin). One thread per (b, d) row; it reads
// everything it needs before writing, so state_out may be state_in.
template <typename T, int W>
__global__ __launch_bounds__(256) void conv_state_kernel(ConvArgs a) {
    constexpr int H = W - 1;
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= a.b * a.d) return;
    const T *xr = static_cast<const T *>(a.xin) + row * a.L;
    float v[H > 0 ? H : 1];
#pragma unroll
    for (int k = 0; k < H; ++k) {
        const int64_t t = a.L - H + k;  // position in the extended sequence, relative to t = 0
        v[k] = t >= 0 ? widen(xr[t]) : (a.state_in ? a.state_in[row * H + (H + t)] : 0.0f);
    }
#pragma unroll
    for (int k = 0; k < H; ++k) a.state_out[row * H + k] = v[k];
}

// Decode: one new input per (b, d): u = c + Σ_{k<W−1} w[k]·state[k] + w[W−1]·xin; the state shifts by one.
template <typename T, int W>
__global__ __launch_bounds__(256) void conv_step_kernel(float *__restrict__ state, const void *xin_, const float *w,
                                                        const float *bias, void *xout_, int64_t bd, int64_t d,
                                                        int silu_on) {
    constexpr int H = W - 1;
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= bd) return;
    const int64_t ch = row % d;
    const float xt = widen(static_cast<const T *>(xin_)[row]);
    float s[H > 0 ? H : 1];
#pragma unroll
    for (int k = 0; k < H; ++k) s[k] = state[row * H + k];
    float u = bias ? bias[ch] : 0.0f;
#pragma unroll
    for (int k = 0; k < H; ++k) u = __builtin_fmaf(w[ch * W + k], s[k], u);
    u = __builtin_fmaf(w[ch * W + H], xt, u);
#pragma unroll
    for (int k = 0; k + 1 < H; ++k) state[row * H + k] = s[k + 1];
    if constexpr (H > 0) state[row * H + H - 1] = xt;
    static_cast<T *>(xout_)[row] = narrow<T>(silu_on ? silu(u) : u);
}

template <typename T, int W>
hipError_t conv_typed(ConvArgs a, hipStream_t stream) {
    constexpr int E = Chunk<T>::kElems;
    const int64_t nch = (a.L + E - 1) / E;
    a.tiles_per_row = (nch + kConvBlock - 1) / kConvBlock;
    a.n_blocks = a.b * a.d * a.tiles_per_row;
    a.fuse_state = a.state_out && a.state_out != a.state_in && a.L >= W - 1 && a.n_blocks > 0;
    if (a.n_blocks > 0) {
        const int64_t grid = a.n_blocks < (int64_t(1) << 30) ? a.n_blocks : (int64_t(1) << 30);
        hipLaunchKernelGGL((conv1d_kernel<T, W>), dim3((unsigned)grid), dim3(kConvBlock), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.state_out && W > 1 && !a.fuse_state) {
        hipLaunchKernelGGL((conv_state_kernel<T, W>), dim3((unsigned)((a.b * a.d + 255) / 256)), dim3(256), 0, stream,
                           a);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename T>
hipError_t conv_dispatch(const ConvArgs &a, int W, hipStream_t stream) {
    switch (W) {
        case 1: return conv_typed<T, 1>(a, stream);
        case 2: return conv_typed<T, 2>(a, stream);
        case 3: return conv_typed<T, 3>(a, stream);
        case 4: return conv_typed<T, 4>(a, stream);
        case 5: return conv_typed<T, 5>(a, stream);
        case 6: return conv_typed<T, 6>(a, stream);
        case 7: return conv_typed<T, 7>(a, stream);
        case 8: return conv_typed<T, 8>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t conv_step_dispatch(const ConvStepLaunch &p, hipStream_t stream) {
    const int64_t bd = p.b * p.d;
    const dim3 grid((unsigned)((bd + 255) / 256)), block(256);
#define SSM_CSTEP(W_) \
    case W_: hipLaunchKernelGGL((conv_step_kernel<T, W_>), grid, block, 0, stream, p.state, p.xin, p.w, p.bias, p.xout, bd, p.d, p.silu_on); break;
    switch (p.W) {
        SSM_CSTEP(1) SSM_CSTEP(2) SSM_CSTEP(3) SSM_CSTEP(4) SSM_CSTEP(5) SSM_CSTEP(6) SSM_CSTEP(7) SSM_CSTEP(8)
        default: return hipErrorInvalidValue;
    }
#undef SSM_CSTEP
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv1d(const ConvLaunch &p, hipStream_t stream) {
    ConvArgs a{};
    a.xin = p.xin; a.w = p.w; a.bias = p.bias; a.state_in = p.state_in; a.xout = p.xout; a.state_out = p.state_out;
    a.b = p.b; a.d = p.d; a.L = p.L; a.silu_on = p.silu_on;
    const int64_t es = p.bf16 ? 2 : 4;
    auto al16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
    a.vec = ((p.L * es) % 16 == 0) && al16(p.xin) && al16(p.xout);
    if (p.bf16) return conv_dispatch<uint16_t>(a, p.W, stream);
    return conv_dispatch<float>(a, p.W, stream);
}

hipError_t launch_conv_step(const ConvStepLaunch &p, hipStream_t stream) {
    if (p.bf16) return conv_step_dispatch<uint16_t>(p, stream);
    return conv_step_dispatch<float>(p, stream);
}

}  // namespace ssm
