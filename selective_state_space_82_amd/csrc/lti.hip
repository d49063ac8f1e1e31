// lti.hip — the time-invariant (LTI) form of the SSM, evaluated as a convolution through the FFT.
//
// Page "State Space Models（SSM）とMamba" §2.3, and page "Mambaとは？Transformer以外の系列モデル", section
// 固定SSMには「再帰」と「畳み込み」の二つの顔がある: when Ā, B̄ and C are the same at every step, the
// zero-state recurrence unrolls into y = x ∗ K̄ with K̄ = (CB̄, CĀB̄, CĀ²B̄, …), K̄ can be computed ahead,
// and the convolution costs O(L log L) through the FFT. Here every channel d is its own system with a
// diagonal A[d][·], B[d][·], C[d][·] and step Δ_d, so K̄_d[k] = Σ_n C_n B̄_n Ā_n^k.
//
// Two kernels:
//   lti_kernel_kernel     K̄ [d][L] fp32, eight consecutive taps per thread: Ā^k from 2^{k·Δ·a·log2 e}.
//   lti_fft_conv_kernel   y = x ∗ K̄ + D·x (· silu(z)), one workgroup per channel. D is folded into the
//                         kernel's first tap (y_t = Σ_s K'_{t−s} x_s with K'_0 = K̄_0 + D). Two batch rows
//                         of the channel share one complex transform (x_b1 + i·x_b2; K̄ is real, so the
//                         real and imaginary parts of the result are the two rows' outputs). The
//                         transform has M = 2^LOGM ≥ 2L points (zero padding makes the circular
//                         convolution linear on the first L outputs).
//
// The transform (M/16 threads, 16 complex values per thread): a decimation-in-frequency forward pass
// sequence (natural order in, digit-reversed out) and its exact inverse, a decimation-in-time sequence
// with conjugate roots (digit-reversed in, natural out), so no reordering is ever done: the product
// with K̄'s spectrum is taken in the digit-reversed order both forward transforms leave behind, in
// registers. Each pass is one radix-R step on groups of R values a span apart, with the in-group DFT in
// registers (radix-2 stages) and the values exchanged through LDS between passes. The first forward
// pass takes its inputs straight from global memory and the last inverse pass hands its outputs straight
// to the epilogue. Twiddles W_M^i = e^{−2πi·i/M} come from two small LDS tables (W_M^{64j} and W_M^{j},
// j < 64, filled with sincospi at the start) and products of their entries.
#include "device_common.h"
#include "launch.h"
#include "ssm_scan.h"
#include "tile_common.h"

namespace ssm {
namespace {

struct LtiKernelArgs {
    const float *delta, *A, *B, *C;
    float *K;
    int64_t d, L, N, blocks_per_channel, n_blocks;
};

constexpr int kKgenPerThread = 8;  // consecutive taps per thread

// One workgroup covers 256·8 consecutive taps of one channel: the channel's per-state constants
// (Ā = 2^u, cb = C·B̄) are formed once into LDS, then each thread takes 2^{k0·u} once per state and
// walks its 8 taps by products (at most 7 roundings from the exponential).
__global__ __launch_bounds__(256) void lti_kernel_kernel(LtiKernelArgs a) {
    __shared__ float s_u[SSM_MAX_N], s_cb[SSM_MAX_N];
    for (int64_t blk = blockIdx.x; blk < a.n_blocks; blk += gridDim.x) {
        const int64_t id = blk / a.blocks_per_channel;  // uniform across the workgroup
        const int64_t k0 = ((blk - id * a.blocks_per_channel) * 256 + threadIdx.x) * kKgenPerThread;
        __syncthreads();  // the previous channel's constants are no longer read
        if (threadIdx.x < a.N) {
            const int64_t n = threadIdx.x;
            const float dt = a.delta[id];
            const float an = a.A[id * a.N + n];
            const float u = dt * (an * kLog2e);
            const float abar = exp2_fast(u);
            s_u[n] = u;
            s_cb[n] = a.C[id * a.N + n] * (zoh_input_coef_log2(dt, u, abar, 1.0f / an) * a.B[id * a.N + n]);
        }
        __syncthreads();
        if (k0 >= a.L) continue;
        float acc[kKgenPerThread] = {};
        for (int n = 0; n < (int)a.N; ++n) {
            const float u = s_u[n];
            float p = s_cb[n] * exp2_fast((float)k0 * u);  // k0 < 2^24: exact
            const float step = exp2_fast(u);
#pragma unroll
            for (int j = 0; j < kKgenPerThread; ++j) {
                acc[j] += p;
                p *= step;
            }
        }
        float *Kd = a.K + id * a.L;
        if (k0 + kKgenPerThread <= a.L && (a.L % 4) == 0 && (reinterpret_cast<uintptr_t>(a.K) & 15) == 0) {
#pragma unroll
            for (int j = 0; j < kKgenPerThread; j += 4)
                *reinterpret_cast<float4 *>(Kd + k0 + j) = make_float4(acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
        } else {
#pragma unroll
            for (int j = 0; j < kKgenPerThread; ++j)
                if (k0 + j < a.L) Kd[k0 + j] = acc[j];
        }
    }
}

// ---- complex helpers ----------------------------------------------------------------------------
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(__builtin_fmaf(a.x, b.x, -a.y * b.y), __builtin_fmaf(a.x, b.y, a.y * b.x));
}
// a · conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
    return make_float2(__builtin_fmaf(a.x, b.x, a.y * b.y), __builtin_fmaf(a.y, b.x, -a.x * b.y));
}

// v · W_16^k (or · conj(W_16^k) when INV), W_16 = e^{−2πi/16}, k in [0, 8); k is a constant after
// unrolling, so the switch folds away.
template <bool INV>
__device__ __forceinline__ float2 rot16(float2 v, int k) {
    constexpr float c1 = 0.92387953251128676f;  // cos(π/8)
    constexpr float s1 = 0.38268343236508977f;  // sin(π/8)
    constexpr float h = 0.70710678118654752f;   // cos(π/4)
    float2 w;
    switch (k) {
        case 0: return v;
        case 4: return INV ? make_float2(-v.y, v.x) : make_float2(v.y, -v.x);  // · (±i)
        case 1: w = make_float2(c1, -s1); break;
        case 2: w = make_float2(h, -h); break;
        case 3: w = make_float2(s1, -c1); break;
        case 5: w = make_float2(-s1, -c1); break;
        case 6: w = make_float2(-h, -h); break;
        default: w = make_float2(-c1, -s1); break;  // 7
    }
    return INV ? cmulc(v, w) : cmul(v, w);
}

constexpr int bitrev(int i, int R) {
    int r = 0;
    for (int m = 1; m < R; m <<= 1) r = (r << 1) | ((i & m) ? 1 : 0);
    return r;
}

// DFT of R values in registers by radix-2 decimation in frequency: natural order in, bit-reversed out.
template <int R>
__device__ __forceinline__ void dft_dif(float2 *v) {
#pragma unroll
    for (int h = R / 2; h >= 1; h >>= 1)
#pragma unroll
        for (int blk = 0; blk < R; blk += 2 * h)
#pragma unroll
            for (int i = 0; i < h; ++i) {
                const float2 p = v[blk + i], q = v[blk + i + h];
                v[blk + i] = cadd(p, q);
                v[blk + i + h] = rot16<false>(csub(p, q), i * (8 / h));
            }
}

// Inverse DFT (conjugate roots, no 1/R) of R values by radix-2 decimation in time: bit-reversed in,
// natural out. Undoes dft_dif up to the factor R.
template <int R>
__device__ __forceinline__ void idft_dit(float2 *v) {
#pragma unroll
    for (int h = 1; h < R; h <<= 1)
#pragma unroll
        for (int blk = 0; blk < R; blk += 2 * h)
#pragma unroll
            for (int i = 0; i < h; ++i) {
                const float2 p = v[blk + i], q = rot16<true>(v[blk + i + h], i * (8 / h));
                v[blk + i] = cadd(p, q);
                v[blk + i + h] = csub(p, q);
            }
}

// LDS index with one pad slot every 16 values (keeps the stride-16 accesses of the short passes off a
// single bank). For a span Q that is 1 or a multiple of 16 and a group start g with g % 16 + 15·Q < 16
// when Q == 1 (groups of 16 aligned to 16), pad(g + j·Q) = pad(g) + j·padded_stride(Q): the group's
// values sit at constant offsets from one address.
__device__ __forceinline__ int pad(int e) { return e + (e >> 4); }
constexpr int padded_stride(int Q) { return Q == 1 ? 1 : Q + Q / 16; }

template <int LOGM>
struct Fft {
    static constexpr int M = 1 << LOGM;
    static constexpr int NT = M / 16;                               // threads
    static constexpr int R0 = (LOGM % 4) == 0 ? 16 : (1 << (LOGM % 4));  // radix of the widest pass
    static constexpr int G0 = 16 / R0;                              // its groups per thread
    static constexpr int Q0 = M / R0;                               // its span between group values
    static constexpr int PADDED = M + M / 16;

    float2 *buf, *tw_hi, *tw_lo;
    int tid;

    // W_M^i for 0 <= i < M
    __device__ __forceinline__ float2 tw(int i) const { return cmul(tw_hi[i >> 6], tw_lo[i & 63]); }

    // v[bitrev(k)] ·= W_M^{idx·k} (CONJ: its conjugate) for 0 < k < R, idx·(R−1) < M. The powers are
    // built one product at a time from W_M^{idx}, restarting from a table value every fourth k, so at
    // most three roundings separate any of them from its exact value and only two stay live.
    template <int R, bool CONJ>
    __device__ __forceinline__ void twiddle(float2 *v, int idx) const {
        if constexpr (R > 1) {
            const float2 w1 = tw(idx);
            float2 wk = w1;
#pragma unroll
            for (int k = 1; k < R; ++k) {
                if (k % 4 == 0) wk = tw(k * idx);
                else if (k > 1) wk = cmul(wk, w1);
                float2 &t = v[bitrev(k, R)];
                t = CONJ ? cmulc(t, wk) : cmul(t, wk);
            }
        }
    }

    // Position of register slot s (= u·R0 + j) in the widest pass: group u of this thread, value j.
    __device__ __forceinline__ int wide_pos(int s) const {
        const int u = s / R0, j = s % R0;
        return tid + NT * (u + j * G0);
    }

    // Forward, widest pass: v holds the natural-order inputs at wide_pos(s); writes to LDS.
    __device__ __forceinline__ void fwd_wide(float2 *v) const {
#pragma unroll
        for (int u = 0; u < G0; ++u) {
            float2 *g = v + u * R0;
            const int r = tid + NT * u;
            dft_dif<R0>(g);
            twiddle<R0, false>(g, r);
            float2 *p = buf + pad(r);
#pragma unroll
            for (int i = 0; i < R0; ++i) p[bitrev(i, R0) * padded_stride(Q0)] = g[i];
        }
    }

    // Forward radix-16 pass with span 16·Q between group values' blocks; Q > 1 goes LDS → LDS,
    // Q == 1 (the last) leaves the digit-reversed result in v.
    template <int Q>
    __device__ __forceinline__ void fwd16(float2 *v) const {
        const int r = tid % Q, base = (tid / Q) * (16 * Q) + r;
        float2 *p = buf + pad(base);
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = p[j * padded_stride(Q)];
        dft_dif<16>(v);
        if constexpr (Q > 1) {
            twiddle<16, false>(v, r * (M / (16 * Q)));
#pragma unroll
            for (int i = 0; i < 16; ++i) p[bitrev(i, 16) * padded_stride(Q)] = v[i];
        }
    }

    // Inverse radix-16 pass, the mirror of fwd16<Q>: Q == 1 takes v (digit-reversed) from registers.
    template <int Q>
    __device__ __forceinline__ void inv16(float2 *v) const {
        const int r = tid % Q, base = (tid / Q) * (16 * Q) + r;
        float2 *p = buf + pad(base);
        if constexpr (Q > 1) {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = p[bitrev(i, 16) * padded_stride(Q)];
            twiddle<16, true>(v, r * (M / (16 * Q)));
        }
        idft_dit<16>(v);
#pragma unroll
        for (int j = 0; j < 16; ++j) p[j * padded_stride(Q)] = v[j];
    }

    // Inverse, widest pass: reads LDS, leaves natural-order outputs at wide_pos(s) in v.
    __device__ __forceinline__ void inv_wide(float2 *v) const {
#pragma unroll
        for (int u = 0; u < G0; ++u) {
            float2 *g = v + u * R0;
            const int r = tid + NT * u;
            const float2 *p = buf + pad(r);
#pragma unroll
            for (int i = 0; i < R0; ++i) g[i] = p[bitrev(i, R0) * padded_stride(Q0)];
            twiddle<R0, true>(g, r);
            idft_dit<R0>(g);
        }
    }

    // Radix-16 passes below the widest one, spans Q0/16, Q0/256, …, 1.
    template <int Q>
    __device__ __forceinline__ void fwd_rest(float2 *v) const {
        fwd16<Q>(v);
        if constexpr (Q > 1) {
            __syncthreads();
            fwd_rest<Q / 16>(v);
        }
    }
    template <int Q>
    __device__ __forceinline__ void inv_rest(float2 *v) const {
        if constexpr (Q > 1) {
            inv_rest<Q / 16>(v);
            __syncthreads();
        }
        inv16<Q>(v);
    }

    // Full forward transform of v (natural order at wide_pos) into v (digit-reversed, registers).
    __device__ __forceinline__ void forward(float2 *v) const {
        fwd_wide(v);
        __syncthreads();
        fwd_rest<Q0 / 16>(v);
    }
    // Full inverse transform (times M) of v (digit-reversed, registers) into v (natural, wide_pos).
    __device__ __forceinline__ void inverse(float2 *v) const {
        inv_rest<Q0 / 16>(v);
        __syncthreads();
        inv_wide(v);
    }
};

struct LtiConvArgs {
    const void *x, *z;
    const float *K, *D;
    void *y;
    int64_t b, d, L;
    // chunked form: `chunk` > 0 steps per transform, n_chunks of them; h_in, delta, A, C as in LtiConvLaunch
    int64_t chunk, n_chunks;
    const float *h_in, *delta, *A, *C;
    int64_t N;
    // items (batch row, chunk) of a channel, b·n_chunks of them in that order, handled by one workgroup:
    // its K̄ spectrum is formed once and serves all of them (two per transform)
    int64_t items_per_wg;
};

// RESP: the chunked form, whose chunks after the first add the response of the state entering them (a
// separate instantiation: the response's loop in the epilogue costs the single-transform form registers).
template <typename T, int LOGM, bool RESP>
// At most 128 VGPRs (four wavefronts per SIMD), so that four workgroups of 256 threads or two of 512 share
// a CU; measured: without the bound, 2^13 points ran at 178 VGPRs, one workgroup per CU, and 1.7× slower.
__global__ __launch_bounds__((1 << LOGM) / 16, 4) void lti_fft_conv_kernel(LtiConvArgs a) {
    using F = Fft<LOGM>;
    constexpr int M = F::M;
    __shared__ float2 s_buf[F::PADDED];
    __shared__ float2 s_hi[M / 64], s_lo[64];
    F f{s_buf, s_hi, s_lo, (int)threadIdx.x};

    // twiddle tables: s_hi[j] = W_M^{64 j}, s_lo[j] = W_M^{j}
    for (int j = threadIdx.x; j < M / 64 + 64; j += F::NT) {
        const int i = j < M / 64 ? 64 * j : j - M / 64;
        float s, c;
        sincospif(2.0f * (float)i / (float)M, &s, &c);  // 2i/M is exact
        (j < M / 64 ? s_hi[j] : s_lo[j - M / 64]) = make_float2(c, -s);
    }
    // workgroup -> (channel id, group g of its items); an item is (batch row, chunk), and one chunk spans
    // the whole sequence when the form is not chunked
    const int64_t id = blockIdx.x % a.d;
    const int64_t g = blockIdx.x / a.d;
    const int64_t klen = a.chunk > 0 ? a.chunk : a.L;  // taps of K per channel
    const int64_t nch = RESP ? a.n_chunks : 1;  // the single-transform form has one chunk per row
    const int64_t i_begin = g * a.items_per_wg;
    const int64_t i_end = (a.b * nch - i_begin) < a.items_per_wg ? a.b * nch : i_begin + a.items_per_wg;
    // chunks after the first add the response of the state entering them: the log2 decays u_n and, per
    // item of the pair, w_n = C_n·h_n (0 for a first chunk)
    __shared__ float s_u[RESP ? SSM_MAX_N : 1], s_w[2][RESP ? SSM_MAX_N : 1];
    if (RESP && threadIdx.x < a.N) {
        const int64_t n = threadIdx.x;
        s_u[n] = a.delta[id] * (a.A[id * a.N + n] * kLog2e);
    }
    __syncthreads();

    // taps of K̄ (and, in the single-transform form, steps). t00 is 0 there (one workgroup per channel); the
    // expressions keep the shape under which that form's kernels fit 128 registers without spilling (a
    // plainer min(L, klen) cost the 2^13-point bf16 kernel two spilled registers and 3.5 %)
    const int64_t t00 = RESP ? 0 : (blockIdx.x / a.d) * klen;
    const int kl = (int)((a.L - t00) < klen ? (a.L - t00) : klen);
    // spectrum of K' (K̄ with D added to its first tap), kept in registers
    float2 kf[16];
    {
        const float dsk = a.D ? a.D[id] : 0.0f;
#pragma unroll
        for (int s = 0; s < 16; ++s) kf[s] = make_float2(0.0f, 0.0f);
        const float *Kd = a.K + id * klen;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int e = f.wide_pos(s);
            if (e < kl) kf[s].x = Kd[e];
        }
        if (threadIdx.x == 0) kf[0].x += dsk;  // wide_pos(0) of thread 0 is position 0
        f.forward(kf);
    }

    const T *xg = static_cast<const T *>(a.x);
    const T *zg = static_cast<const T *>(a.z);
    T *yg = static_cast<T *>(a.y);
    constexpr float inv_m = 1.0f / (float)M;
    if constexpr (!RESP) {  // one transform per row pair: the batch rows of the pair share the chunk
        for (int64_t b1 = 0; b1 < a.b; b1 += 2) {
            const bool two = b1 + 1 < a.b;
            // the pair's rows (workgroup-uniform pointers; per-lane offsets stay 32-bit)
            const T *x1 = xg + (b1 * a.d + id) * a.L + t00;
            const T *x2 = two ? x1 + a.d * a.L : x1;
            float2 v[16];
    #pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int e = f.wide_pos(s);
                const bool in = e < kl;
                v[s] = make_float2(in ? widen(x1[e]) : 0.0f, in && two ? widen(x2[e]) : 0.0f);
            }
            __syncthreads();  // the previous pair's last reads of s_buf (and s_w) are done
            f.forward(v);
    #pragma unroll
            for (int s = 0; s < 16; ++s) v[s] = cmul(v[s], kf[s]);
            f.inverse(v);
            const int64_t o1 = (b1 * a.d + id) * a.L + t00;
            const int64_t o2 = two ? o1 + a.d * a.L : o1;
            T *y1p = yg + o1, *y2p = yg + o2;
            const T *z1 = zg ? zg + o1 : nullptr, *z2 = zg ? zg + o2 : nullptr;
    #pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int e = f.wide_pos(s);
                if (e < kl) {
                    float y1 = v[s].x * inv_m, y2 = v[s].y * inv_m;
                    if (zg) {
                        y1 *= silu(widen(z1[e]));
                        if (two) y2 *= silu(widen(z2[e]));
                    }
                    y1p[e] = narrow<T>(y1);
                    if (two) y2p[e] = narrow<T>(y2);
                }
            }
        }
    } else {  // the chunked form: the workgroup's items (batch row, chunk), two per transform
        // the pair's items (batch row, chunk), stepped along without divisions (a 64-bit division per pair
        // held enough registers to make this instantiation spill in its transform loop)
        int64_t b1 = i_begin / nch, j1 = i_begin - b1 * nch;
        for (int64_t i1 = i_begin; i1 < i_end; i1 += 2) {
            const bool two = i1 + 1 < i_end;
            int64_t bn = b1, jn = j1 + 1;  // item i1 + 1
            if (jn == nch) { jn = 0; ++bn; }
            const int64_t b2 = two ? bn : b1, j2 = two ? jn : j1;
            const int64_t t01 = j1 * klen, t02 = j2 * klen;
            const int L1 = (int)((a.L - t01) < klen ? (a.L - t01) : klen);
            const int L2 = two ? (int)((a.L - t02) < klen ? (a.L - t02) : klen) : 0;
            // the pair's rows (workgroup-uniform pointers; per-lane offsets stay 32-bit)
            const T *x1 = xg + (b1 * a.d + id) * a.L + t01;
            const T *x2 = xg + (b2 * a.d + id) * a.L + t02;
            float2 v[16];
    #pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int e = f.wide_pos(s);
                v[s] = make_float2(e < L1 ? widen(x1[e]) : 0.0f, e < L2 ? widen(x2[e]) : 0.0f);
            }
            __syncthreads();  // the previous pair's last reads of s_buf (and s_w) are done
            if (RESP && threadIdx.x < a.N) {
                const int64_t n = threadIdx.x;
                const float cn = a.C[id * a.N + n];
                s_w[0][n] = j1 > 0 ? cn * a.h_in[((b1 * a.d + id) * (nch - 1) + (j1 - 1)) * a.N + n] : 0.0f;
                s_w[1][n] = j2 > 0 && two ? cn * a.h_in[((b2 * a.d + id) * (nch - 1) + (j2 - 1)) * a.N + n] : 0.0f;
            }
            f.forward(v);
    #pragma unroll
            for (int s = 0; s < 16; ++s) v[s] = cmul(v[s], kf[s]);
            f.inverse(v);
            if (RESP) {
                // + M·Σ_n w_n·Ā_n^{e+1} on the unscaled outputs (M is a power of 2, so the later 1/M is exact).
                // This thread's positions are e = tid + NT·k (k = 0 .. 15, slot (k % G0)·R0 + k / G0), so the
                // powers form a geometric sequence in k: Ā^{tid+1} and the ratio Ā^{NT}, one exp each per state,
                // then a product per position (at most 15 products: about 16 ulp). s_w was written before the
                // transforms' barriers.
                const float e0 = (float)(threadIdx.x + 1);
    #pragma unroll 1
                for (int n = 0; n < (int)a.N; ++n) {
                    const float un = s_u[n];
                    const float w1 = s_w[0][n] * (float)M, w2 = s_w[1][n] * (float)M;
                    float pw = exp2_fast(e0 * un);
                    const float q = exp2_fast((float)F::NT * un);
    #pragma unroll
                    for (int k = 0; k < 16; ++k) {
                        const int sl = (k % F::G0) * F::R0 + k / F::G0;
                        v[sl].x = __builtin_fmaf(w1, pw, v[sl].x);
                        v[sl].y = __builtin_fmaf(w2, pw, v[sl].y);
                        pw *= q;
                    }
                }
            }
            const int64_t o1 = (b1 * a.d + id) * a.L + t01;
            const int64_t o2 = (b2 * a.d + id) * a.L + t02;
            T *y1p = yg + o1, *y2p = yg + o2;
            const T *z1 = zg ? zg + o1 : nullptr, *z2 = zg ? zg + o2 : nullptr;
    #pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int e = f.wide_pos(s);
                if (e < L1) {
                    float y1 = v[s].x * inv_m;
                    if (zg) y1 *= silu(widen(z1[e]));
                    y1p[e] = narrow<T>(y1);
                }
                if (e < L2) {
                    float y2 = v[s].y * inv_m;
                    if (zg) y2 *= silu(widen(z2[e]));
                    y2p[e] = narrow<T>(y2);
                }
            }
            b1 = bn;  // item i1 + 2
            j1 = jn + 1;
            if (j1 == nch) { j1 = 0; ++b1; }
        }
    }
}

template <typename T, int LOGM>
hipError_t launch_conv_m(const LtiConvArgs &a, hipStream_t stream) {
    const int64_t groups = (a.b * a.n_chunks + a.items_per_wg - 1) / a.items_per_wg;
    const dim3 grid((unsigned)(a.d * groups)), block((1 << LOGM) / 16);
    if (a.h_in) {
        if constexpr ((int64_t(1) << LOGM) == 2 * kLtiChunk) {
            hipLaunchKernelGGL((lti_fft_conv_kernel<T, LOGM, true>), grid, block, 0, stream, a);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;  // the chunked form uses one transform size
    }
    hipLaunchKernelGGL((lti_fft_conv_kernel<T, LOGM, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

// End state of chunk j of row (b, d) from zero, for chunks 0 .. n_chunks − 2 (all of full length):
// E_n = B̄_n·Σ_s Ā_n^{chunk−1−s}·x_s. One wavefront per (row, chunk): lane l takes the 64 consecutive steps
// 64 l .. 64 l + 63 (16-byte loads) by Horner's rule (acc ← acc·Ā + x, so no power is formed), for 16 states
// at a time, and scales its sum by Ā^{chunk−64(l+1)} (one exp per state). The 64 lanes' sums of the 16
// states are then added by a transposing butterfly: at each of the first four exchanges a lane keeps half of
// the states it still holds and hands the other half to its partner, so 8 + 4 + 2 + 1 + 2 = 17 exchanges
// leave lane l with the whole sum of one state (15 of them per state at one exchange per state and step).
template <typename T>
__global__ __launch_bounds__(kWave) void lti_chunk_agg_kernel(LtiChunkLaunch p, int64_t n_chunks, int vec) {
    constexpr int kPer = 64;                        // steps per lane
    constexpr int E = Chunk<T>::kElems;
    constexpr int kG = 16;                          // states per group
    const int64_t nc1 = n_chunks - 1;
    const int64_t row = blockIdx.x / nc1;           // b·d + d
    const int64_t j = blockIdx.x - row * nc1;
    const int64_t id = row % p.d;
    const int lane = threadIdx.x;
    const T *xr = static_cast<const T *>(p.x) + row * p.L + j * p.chunk;
    const int64_t s0 = (int64_t)lane * kPer;
    uint4 xv[kPer / E];
#pragma unroll
    for (int q = 0; q < kPer / E; ++q) xv[q] = get_chunk<T>(xr, s0 + q * E, p.chunk, s0 < p.chunk, vec != 0);
    const float dt = p.delta[id];
    const bool in = s0 < p.chunk;                     // chunk is a multiple of kPer: a lane is wholly in or out
    const float rest = in ? (float)(p.chunk - kPer - s0) : 0.0f;  // steps after this lane's last one
    for (int n0 = 0; n0 < (int)p.N; n0 += kG) {
        float u[kG], ab[kG], acc[kG];
#pragma unroll
        for (int i = 0; i < kG; ++i) {
            const int n = n0 + i;
            u[i] = n < (int)p.N ? dt * (p.A[id * p.N + n] * kLog2e) : 0.0f;
            ab[i] = exp2_fast(u[i]);
            acc[i] = 0.0f;
        }
#pragma unroll
        for (int q = 0; q < kPer / E; ++q) {
            float xs[E];
            chunk_to_regs<T>(xs, xv[q]);
#pragma unroll
            for (int e = 0; e < E; ++e) {
#pragma unroll
                for (int i = 0; i < kG; ++i) acc[i] = __builtin_fmaf(acc[i], ab[i], xs[e]);
            }
        }
#pragma unroll
        for (int i = 0; i < kG; ++i) acc[i] = in ? acc[i] * exp2_fast(rest * u[i]) : 0.0f;
        // transposing butterfly over the lanes: exchange across lane bit m keeps the lower half of the
        // states held when that bit is 0, the upper half when it is 1
#pragma unroll
        for (int h = kG / 2, m = 32; h >= 1; h /= 2, m /= 2) {
            const bool up = (lane & m) != 0;
#pragma unroll
            for (int i = 0; i < h; ++i) {
                const float keep = up ? acc[h + i] : acc[i];
                const float give = up ? acc[i] : acc[h + i];
                acc[i] = keep + __shfl_xor(give, m);
            }
        }
        acc[0] += __shfl_xor(acc[0], 2);
        acc[0] += __shfl_xor(acc[0], 1);
        // lane l now holds state n0 + 8·bit5 + 4·bit4 + 2·bit3 + bit2 of l
        const int n = n0 + ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
        if ((lane & 3) == 0 && n < (int)p.N) {
            const float an = p.A[id * p.N + n];
            const float un = dt * (an * kLog2e);
            p.H[(row * nc1 + j) * p.N + n] = acc[0] * (zoh_input_coef_log2(dt, un, exp2_fast(un), 1.0f / an) * p.B[id * p.N + n]);
        }
    }
}

// The states between chunks, in place: H_j ← Ā^chunk·H_{j−1} + H_j per (row, n), walking the chunks in order.
__global__ __launch_bounds__(256) void lti_chunk_carry_kernel(LtiChunkLaunch p, int64_t n_chunks) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (row, n)
    if (i >= p.b * p.d * p.N) return;
    const int64_t row = i / p.N, n = i - row * p.N, id = row % p.d;
    const float pc = exp2_fast((float)p.chunk * (p.delta[id] * (p.A[id * p.N + n] * kLog2e)));
    const int64_t nc1 = n_chunks - 1;
    float *h = p.H + row * nc1 * p.N + n;
    float acc = 0.0f;
    for (int64_t j = 0; j < nc1; ++j) {
        acc = __builtin_fmaf(pc, acc, h[j * p.N]);
        h[j * p.N] = acc;
    }
}

template <typename T>
hipError_t launch_conv_typed(const LtiConvArgs &a, int logm, hipStream_t stream) {
    switch (logm) {
        case 10: return launch_conv_m<T, 10>(a, stream);
        case 11: return launch_conv_m<T, 11>(a, stream);
        case 12: return launch_conv_m<T, 12>(a, stream);
        case 13: return launch_conv_m<T, 13>(a, stream);
        case 14: return launch_conv_m<T, 14>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int lti_fft_log2(int64_t L) {
    int logm = kLtiMinLog2;
    while ((int64_t(1) << logm) < 2 * L) ++logm;
    return logm;
}

hipError_t launch_lti_kernel(const LtiKernelLaunch &p, hipStream_t stream) {
    if (p.d == 0 || p.L == 0) return hipSuccess;
    constexpr int64_t per_block = 256 * kKgenPerThread;
    LtiKernelArgs a{p.delta, p.A, p.B, p.C, p.K, p.d, p.L, p.N, (p.L + per_block - 1) / per_block, 0};
    a.n_blocks = p.d * a.blocks_per_channel;
    const int64_t grid = a.n_blocks < (int64_t(1) << 30) ? a.n_blocks : (int64_t(1) << 30);
    hipLaunchKernelGGL(lti_kernel_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_lti_conv(const LtiConvLaunch &p, hipStream_t stream) {
    if (p.b == 0 || p.d == 0 || p.L == 0) return hipSuccess;
    const int64_t klen = p.chunk > 0 ? p.chunk : p.L;
    const int64_t n_chunks = (p.L + klen - 1) / klen;
    // the chunked form: up to 32 items (batch row, chunk) per workgroup, an even number so that they pair
    // up, the channel's K̄ spectrum transformed once for all of them; the single-transform form: all batch
    // rows of a channel in one workgroup
    const int64_t items = p.b * n_chunks;
    const int64_t per_wg = n_chunks == 1 ? p.b : (items < 32 ? items + (items & 1) : 32);
    const LtiConvArgs a{p.x, p.z, p.K, p.D, p.y, p.b, p.d, p.L, p.chunk, n_chunks,
                        n_chunks > 1 ? p.h_in : nullptr, p.delta, p.A, p.C, p.N, per_wg};
    if (n_chunks > 1 && (!p.h_in || !p.delta || !p.A || !p.C || p.N < 1 || p.N > SSM_MAX_N)) return hipErrorInvalidValue;
    if (p.d * ((items + per_wg - 1) / per_wg) > 0x7fffffffLL) return hipErrorInvalidValue;
    const int logm = lti_fft_log2(klen);
    if (logm > kLtiMaxLog2) return hipErrorInvalidValue;
    if (p.bf16) return launch_conv_typed<uint16_t>(a, logm, stream);
    return launch_conv_typed<float>(a, logm, stream);
}

hipError_t launch_lti_chunk_states(const LtiChunkLaunch &p, hipStream_t stream) {
    const int64_t n_chunks = (p.L + p.chunk - 1) / p.chunk;
    if (n_chunks <= 1 || p.b == 0 || p.d == 0) return hipSuccess;
    if (p.chunk > 64 * kWave || p.chunk % 64 != 0 || p.N < 1 || p.N > SSM_MAX_N) return hipErrorInvalidValue;
    const int64_t blocks = p.b * p.d * (n_chunks - 1);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    // 16-byte loads when every chunk of every row starts on a 16-byte boundary
    const int64_t esize = p.bf16 ? 2 : 4;
    const int vec = (reinterpret_cast<uintptr_t>(p.x) & 15u) == 0 && (p.L * esize) % 16 == 0 && (p.chunk * esize) % 16 == 0;
    if (p.bf16)
        hipLaunchKernelGGL(lti_chunk_agg_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kWave), 0, stream, p, n_chunks, vec);
    else
        hipLaunchKernelGGL(lti_chunk_agg_kernel<float>, dim3((unsigned)blocks), dim3(kWave), 0, stream, p, n_chunks, vec);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = p.b * p.d * p.N;
    hipLaunchKernelGGL(lti_chunk_carry_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, p, n_chunks);
    return hipGetLastError();
}

}  // namespace ssm
