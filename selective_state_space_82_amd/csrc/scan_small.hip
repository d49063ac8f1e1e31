// scan_small.hip — the prefill of small problems for gfx950: a short sequence on few channel blocks.
//
// Method (page "Mambaとは？Transformer以外の系列モデル", section 状態空間モデルを一つの式から理解する for the
// ZOH terms Ā = e^{ΔA}, B̄ = (e^{ΔA} − 1)/A·B and the recurrence h_t = Ā h_{t−1} + B̄ x_t, y_t = C_t h_t + D x_t;
// section Selective Scanは選択機構そのものではない: the per-step affine maps compose associatively, so a
// sequence can be cut into segments whose maps are formed independently and then chained).
//
// When the whole problem is a few channel blocks over at most kSmallSeg·kSmallMaxWaves steps, the time
// split of the main prefill costs two launches and a rescan that the short sequence does not repay, and
// without it one wavefront walks every step in turn. Here one workgroup holds one block of 16 channels of
// one batch row, and wavefront w takes the `seg` steps from seg·w (8 where 16 wavefronts of 8 cover the
// sequence, else 16):
//   1. every wavefront stages its steps' x, Δ, z and B, C rows in LDS;
//   2. every wavefront but the last forms its segment's map h ↦ P·h + E (E its end state from zero,
//      P = e^{A·ΣΔ}) and leaves it in LDS;
//   3. after one barrier, wavefront w chains the maps of the segments before it onto the initial state and
//      walks its own steps from that state, reading out y, and the last one stores the final state.
// So the longest chain of dependent steps is twice `seg` instead of the sequence length.
//
// Lanes: channel c = lane / 4 of the block, states 4·(lane % 4) .. +3 (N <= 16); the readout's partial sums
// of a channel's four lanes are added by two xor exchanges. Arithmetic is the unscaled recurrence with the
// input coefficient from its series where |ΔA| < 1/16 (the decode kernel's), so A = 0 takes the limit Δ·B.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "launch.h"

namespace ssm {
namespace {

constexpr int kCh = kSmallCh;
constexpr int kNS = 16;   // state slots per channel (4 lanes × 4 states)
constexpr float kZeroA = 5.421010862e-20f;  // 2^-64: |A| below this takes the A = 0 limit

struct SmallArgs {
    const void *x, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z;
    void *y;
    float *final_state;
    const float *init_state;
    int64_t b, d, L, N;
    int64_t n_cb;  // blocks of 16 channels per batch row
    int seg;       // steps per wavefront: kSmallSeg / 2 up to kSmallMaxWaves such segments, else kSmallSeg
};

template <typename T>
__global__ __launch_bounds__(kWave * kSmallMaxWaves) void scan_small_kernel(SmallArgs a) {
    constexpr int S = kSmallSeg;  // LDS rows hold up to kSmallSeg steps
    __shared__ __attribute__((aligned(16))) float xs[kSmallMaxWaves][kCh][S];
    __shared__ __attribute__((aligned(16))) float ds[kSmallMaxWaves][kCh][S];
    __shared__ __attribute__((aligned(16))) float zs[kSmallMaxWaves][kCh][S];
    __shared__ __attribute__((aligned(16))) float bs[kSmallMaxWaves][S][kNS];
    __shared__ __attribute__((aligned(16))) float cs[kSmallMaxWaves][S][kNS];
    __shared__ __attribute__((aligned(16))) float sP[kSmallMaxWaves][kCh][kNS];
    __shared__ __attribute__((aligned(16))) float sE[kSmallMaxWaves][kCh][kNS];

    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int c = lane / 4, g = lane % 4;
    const int64_t bi = blockIdx.x / a.n_cb;
    const int64_t ch = (blockIdx.x - bi * a.n_cb) * kCh + c;
    const bool ch_ok = ch < a.d;
    const int N = (int)a.N;
    const int64_t t0 = (int64_t)w * a.seg;
    const int nk = (int)((a.L - t0) < a.seg ? (a.L - t0) : a.seg);  // steps of this wavefront (>= 1)
    const T *xg = static_cast<const T *>(a.x);
    const T *dg = static_cast<const T *>(a.delta);
    const T *zg = static_cast<const T *>(a.z);
    const T *Bg = static_cast<const T *>(a.B) + bi * a.L * a.N;
    const T *Cg = static_cast<const T *>(a.C) + bi * a.L * a.N;
    const int64_t row = bi * a.d + ch;

    // 1. staging: lane (c, g) takes steps 4g .. 4g + 3 of channel c's rows, and (step c, states 4g .. 4g + 3)
    //    of the B and C runs; zeros past the sequence, the channels and the states
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int k = 4 * g + q;
        const bool ok = ch_ok && k < nk;
        const int64_t o = row * a.L + t0 + k;
        xs[w][c][k] = ok ? widen(xg[ok ? o : 0]) : 0.0f;
        ds[w][c][k] = ok ? widen(dg[ok ? o : 0]) : 0.0f;
        zs[w][c][k] = ok && zg ? widen(zg[ok ? o : 0]) : 0.0f;
        const int n = 4 * g + q;
        const bool bok = c < nk && n < N;
        const int64_t bo = (t0 + c) * a.N + n;
        bs[w][c][n] = bok ? widen(Bg[bok ? bo : 0]) : 0.0f;
        cs[w][c][n] = bok ? widen(Cg[bok ? bo : 0]) : 0.0f;
    }

    // this lane's states: log2-scaled A, 1/A (1 at the A = 0 limit), validity
    float a2[4], ia[4], h[4];
    bool zero[4], live[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = 4 * g + j;
        live[j] = ch_ok && n < N;
        const float av = live[j] ? a.A[ch * a.N + n] : -1.0f;
        zero[j] = __builtin_fabsf(av) < kZeroA;
        a2[j] = zero[j] ? 0.0f : av * kLog2e;
        ia[j] = zero[j] ? 1.0f : 1.0f / av;
        h[j] = 0.0f;
    }
    __syncthreads();

    // one step k of this wavefront's segment: h ← Ā h + B̄ x (B is 0 for the states past N)
    auto step = [&](int k) {
        const float dt = ds[w][c][k], xv = xs[w][c][k];
        const float4 bv = *reinterpret_cast<const float4 *>(&bs[w][k][4 * g]);
        const float bj[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float u = dt * a2[j];
            const float ab = exp2_fast(u);
            const float be = zoh_input_coef_log2(dt, u, ab, ia[j]);
            h[j] = __builtin_fmaf(ab, h[j], be * (bj[j] * xv));
        }
        return dt;
    };

    // 2. the segment's map, for every wavefront but the last
    const int nw = (int)((a.L + a.seg - 1) / a.seg);
    if (w < nw - 1) {
        float dsum = 0.0f;
        for (int k = 0; k < nk; ++k) dsum += step(k);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sE[w][c][4 * g + j] = h[j];
            sP[w][c][4 * g + j] = zero[j] ? 1.0f : exp2_fast(a2[j] * dsum);
            h[j] = 0.0f;
        }
    }
    __syncthreads();

    // 3. the entering state, chained from the initial state over the segments before this one
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (live[j] && a.init_state) h[j] = a.init_state[row * a.N + 4 * g + j];
    for (int q = 0; q < w; ++q) {
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = __builtin_fmaf(sP[q][c][4 * g + j], h[j], sE[q][c][4 * g + j]);
    }
    const float dsk = ch_ok && a.D ? a.D[ch] : 0.0f;
    T *yg = static_cast<T *>(a.y);
    for (int k = 0; k < nk; ++k) {
        step(k);
        const float4 cv = *reinterpret_cast<const float4 *>(&cs[w][k][4 * g]);
        float acc = cv.x * h[0];
        acc = __builtin_fmaf(cv.y, h[1], acc);
        acc = __builtin_fmaf(cv.z, h[2], acc);
        acc = __builtin_fmaf(cv.w, h[3], acc);
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        float yv = __builtin_fmaf(dsk, xs[w][c][k], acc);
        if (zg) yv *= silu(zs[w][c][k]);
        if (g == 0 && ch_ok) yg[row * a.L + t0 + k] = narrow<T>(yv);
    }
    if (w == nw - 1 && a.final_state) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (live[j]) a.final_state[row * a.N + 4 * g + j] = h[j];
    }
}

}  // namespace

hipError_t launch_scan_small(const FwdLaunch &p, hipStream_t stream) {
    if (!small_problem(p.b, p.d, p.L, p.N)) return hipErrorInvalidValue;
    SmallArgs a{p.x, p.delta, p.A, p.B, p.C, p.D, p.z, p.y, p.final_state, p.init_state,
                p.b, p.d, p.L, p.N, (p.d + kCh - 1) / kCh};
    a.seg = small_seg(p.L);
    const int waves = (int)((p.L + a.seg - 1) / a.seg);
    const dim3 grid((unsigned)(p.b * a.n_cb)), block((unsigned)(kWave * waves));
    // the dispatch carries the timing events, as the main prefill's output kernel does
    if (p.bf16)
        hipExtLaunchKernelGGL((scan_small_kernel<uint16_t>), grid, block, 0, stream, p.ev_begin, p.ev_end, 0u, a);
    else
        hipExtLaunchKernelGGL((scan_small_kernel<float>), grid, block, 0, stream, p.ev_begin, p.ev_end, 0u, a);
    return hipGetLastError();
}

}  // namespace ssm
