// ssd.hip — the scalar-decay selective SSM (one decay a_h per head of P channels, Δ shared by the head)
// evaluated chunk by chunk with matrix products on the MFMA units.
//
// Page "State Space Models（SSM）とMamba" §4.6 (Mamba-2: state space duality relates SSMs and linear
// attention) together with the unrolled recurrence of page "Mambaとは？Transformer以外の系列モデル", section
// Mambaの核心は入力依存のDelta、B、C: with A = a·I the product of the Ā_r over a span is the scalar
// exp(a Σ Δ_r), so within a chunk of Q steps
//   y_t = Σ_{s<=t in chunk} (C_t·B_s) e^{a(c_t − c_s)} β_s x_s  +  e^{a c_t} C_t·h_in  +  D x_t,
// where c_t = Σ_{r<=t in chunk} Δ_r, β_s the ZOH input coefficient and h_in the state entering the chunk,
// and the state leaving it is h_out = e^{a c_end} h_in + Σ_s e^{a(c_end − c_s)} β_s B_s x_sᵀ. Per (b, head,
// chunk) those are dense products: G = C Bᵀ (Q×Q over N), Y = (G ∘ decay) Xᵀ (Q×P over Q), C H_inᵀ (Q×P over
// N) and the chunk state X_w Bᵀ (P×N over Q), all on v_mfma_f32_32x32x2f32 (fp32 in, fp32 accumulate).
//
// Three kernels:
//   ssd_state_kernel   per (b, h, chunk): the chunk's own state contribution S_c [P][N] and its decay.
//   ssd_pass_kernel    per (b, h, p, n): walks the chunks in order, replacing S_c by the state entering
//                      chunk c and writing the final state.
//   ssd_out_kernel     per (b, h, chunk): the outputs of the chunk from its inputs and entering state.
//
// MFMA 32x32x2 f32 lane layout (checked on the device): lane l supplies A[l % 32][l / 32] and
// B[l / 32][l % 32]; result register r of lane l is D[8(r / 4) + 4(l / 32) + r % 4][l % 32].
#include "device_common.h"
#include "launch.h"

namespace ssm {
namespace {

typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int kQ = 64;           // chunk length
constexpr int kP = 64;           // channels per head
constexpr int kXP = kQ + 1;      // padded row of x [p][s] and of the decayed products [t][s] in LDS
constexpr int kThreads = 256;    // four wavefronts

struct SsdArgs {
    const void *x, *delta, *B, *C, *z;
    const float *A, *D, *h0;
    void *y;
    float *hT;
    float *S;      // [b][H][nc][P][N] chunk states, then entering states
    float *decay;  // [b][H][nc]
    int64_t b, H, L, nc;
};

__device__ __forceinline__ int lane() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave() { return threadIdx.x >> 6; }

// Row position of result register r of lane l in a 32×32 tile.
__device__ __forceinline__ int d_row(int r, int l) { return 8 * (r / 4) + 4 * (l / 32) + (r % 4); }

// Wavefront 0 turns the chunk's Δ into the in-chunk running sum of Δ·a·log2 e (cum, inclusive) and the
// ZOH input coefficient β; steps past L get Δ = 0 (no decay, no input).
template <typename T>
__device__ __forceinline__ void chunk_scalars(const SsdArgs &a, int64_t bh, int64_t t0, float ah, float *s_cum,
                                              float *s_beta) {
    if (wave() != 0) return;
    const int i = lane();
    const T *dg = static_cast<const T *>(a.delta) + bh * a.L;
    const float dt = t0 + i < a.L ? widen(dg[t0 + i]) : 0.0f;
    const float u = dt * (ah * kLog2e);
    const float abar = exp2_fast(u);
    const float beta = zoh_input_coef_log2(dt, u, abar, 1.0f / ah);
    float c = u;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float o = __shfl_up(c, m, 64);
        if (i >= m) c += o;
    }
    s_cum[i] = c;
    s_beta[i] = beta;
}

// Rows [t0, t0 + 64) of a [L][N] tensor of batch row ib into LDS rows of stride N + 1 (zeros past L).
template <typename T, int N>
__device__ __forceinline__ void load_rows_tn(const void *src, int64_t ib, int64_t t0, int64_t L, float *dst) {
    const T *g = static_cast<const T *>(src) + (ib * L + t0) * N;
    for (int idx = threadIdx.x; idx < kQ * N; idx += kThreads) {
        const int t = idx / N, n = idx % N;
        dst[t * (N + 1) + n] = t0 + t < L ? widen(g[idx]) : 0.0f;
    }
}

// x rows of head h, steps [t0, t0 + 64), into LDS [p][s] (stride kXP), each value times w[s] if given.
template <typename T>
__device__ __forceinline__ void load_x(const SsdArgs &a, int64_t ib, int64_t h, int64_t t0, const float *w,
                                       float *dst) {
    const T *g = static_cast<const T *>(a.x) + ((ib * a.H + h) * kP) * a.L;
    for (int idx = threadIdx.x; idx < kP * kQ; idx += kThreads) {
        const int p = idx / kQ, s = idx % kQ;
        float v = t0 + s < a.L ? widen(g[p * a.L + t0 + s]) : 0.0f;
        if (w) v *= w[s];
        dst[p * kXP + s] = v;
    }
}

template <typename T, int N>
__global__ __launch_bounds__(kThreads) void ssd_state_kernel(SsdArgs a) {
    __shared__ float s_cum[kQ], s_beta[kQ], s_w[kQ];
    __shared__ float s_x[kP * kXP];
    __shared__ float s_b[kQ * (N + 1)];
    const int64_t c = blockIdx.x % a.nc, bh = blockIdx.x / a.nc;
    const int64_t ib = bh / a.H, h = bh % a.H;
    const int64_t t0 = c * kQ;
    const float ah = a.A[h];
    chunk_scalars<T>(a, bh, t0, ah, s_cum, s_beta);
    __syncthreads();
    if (threadIdx.x < kQ) {
        const float cend = s_cum[kQ - 1];
        s_w[threadIdx.x] = exp2_fast(cend - s_cum[threadIdx.x]) * s_beta[threadIdx.x];
        if (threadIdx.x == 0) a.decay[bh * a.nc + c] = exp2_fast(cend);
    }
    __syncthreads();
    load_x<T>(a, ib, h, t0, s_w, s_x);
    load_rows_tn<T, N>(a.B, ib, t0, a.L, s_b);
    __syncthreads();
    // S[p][n] = Σ_s x_w[p][s] B[s][n]: 2 × N/32 tiles of 32×32, spread over the four wavefronts
    const int l = lane();
    float *S = a.S + (bh * a.nc + c) * (int64_t)(kP * N);
    for (int tile = wave(); tile < 2 * (N / 32); tile += 4) {
        const int qp = tile % 2, qn = tile / 2;
        f16v acc = {};
#pragma unroll 8
        for (int s0 = 0; s0 < kQ; s0 += 2) {
            const float av = s_x[(32 * qp + l % 32) * kXP + s0 + l / 32];
            const float bv = s_b[(s0 + l / 32) * (N + 1) + 32 * qn + l % 32];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) S[(32 * qp + d_row(r, l)) * N + 32 * qn + l % 32] = acc[r];
    }
}

// One thread per (b, h, p, n): h ← decay_c·h + S_c over the chunks, leaving in S_c the state that enters
// chunk c; the last value is the final state.
template <int N>
__global__ __launch_bounds__(256) void ssd_pass_kernel(SsdArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= a.b * a.H * kP * N) return;
    const int64_t pn = gid % (kP * N), bh = gid / (kP * N);
    float hv = a.h0 ? a.h0[bh * (kP * N) + pn] : 0.0f;  // [b][H·P][N] = [b·H][P·N]
    float *S = a.S + bh * a.nc * (kP * N) + pn;
    const float *dec = a.decay + bh * a.nc;
    for (int64_t c = 0; c < a.nc; ++c) {
        const float s = S[c * (kP * N)];
        S[c * (kP * N)] = hv;
        hv = __builtin_fmaf(dec[c], hv, s);
    }
    if (a.hT) a.hT[bh * (kP * N) + pn] = hv;
}

template <typename T, int N>
__global__ __launch_bounds__(kThreads) void ssd_out_kernel(SsdArgs a) {
    constexpr int CP = N + 1;
    constexpr int BM = (kQ * CP > kQ * kXP) ? kQ * CP : kQ * kXP;
    __shared__ float s_cum[kQ], s_beta[kQ];
    __shared__ float s_c[kQ * CP];  // C [t][n]
    __shared__ float s_bm[BM];      // B [s][n], then the decayed products M [t][s]
    __shared__ float s_h[kP * CP];  // entering state [p][n]
    __shared__ float s_x[kP * kXP]; // x [p][s]
    const int64_t c = blockIdx.x % a.nc, bh = blockIdx.x / a.nc;
    const int64_t ib = bh / a.H, h = bh % a.H;
    const int64_t t0 = c * kQ;
    const float ah = a.A[h];
    chunk_scalars<T>(a, bh, t0, ah, s_cum, s_beta);
    load_rows_tn<T, N>(a.C, ib, t0, a.L, s_c);
    load_rows_tn<T, N>(a.B, ib, t0, a.L, s_bm);
    load_x<T>(a, ib, h, t0, nullptr, s_x);
    {
        const float *Hin = a.S + (bh * a.nc + c) * (int64_t)(kP * N);
        for (int idx = threadIdx.x; idx < kP * N; idx += kThreads) s_h[(idx / N) * CP + idx % N] = Hin[idx];
    }
    __syncthreads();

    const int l = lane(), w = wave();
    // G = C Bᵀ on the three tiles at or below the diagonal, then M = G ∘ e^{a(c_t − c_s)} β_s (s <= t)
    f16v g = {};
    const int qt = w == 0 ? 0 : 1, qs = w == 2 ? 1 : 0;
    if (w < 3) {
#pragma unroll 8
        for (int n0 = 0; n0 < N; n0 += 2) {
            const float av = s_c[(32 * qt + l % 32) * CP + n0 + l / 32];
            const float bv = s_bm[(32 * qs + l % 32) * CP + n0 + l / 32];
            g = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, g, 0, 0, 0);
        }
    }
    __syncthreads();  // B is no longer read: its space takes M
    if (w < 3) {
        const int s = 32 * qs + l % 32;
        const float cs = s_cum[s], bs = s_beta[s];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = 32 * qt + d_row(r, l);
            s_bm[t * kXP + s] = s <= t ? g[r] * exp2_fast(s_cum[t] - cs) * bs : 0.0f;
        }
    }
    __syncthreads();

    // this wavefront's 32×32 output tile: rows t in [32·ot, +32), channels p in [32·op, +32)
    const int ot = w / 2, op = w % 2;
    f16v acc = {};
    const int s_end = 32 * (ot + 1);  // M[t][s] = 0 for s > t
    for (int s0 = 0; s0 < s_end; s0 += 2) {
        const float av = s_bm[(32 * ot + l % 32) * kXP + s0 + l / 32];
        const float bv = s_x[(32 * op + l % 32) * kXP + s0 + l / 32];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    f16v inter = {};
#pragma unroll 8
    for (int n0 = 0; n0 < N; n0 += 2) {
        const float av = s_c[(32 * ot + l % 32) * CP + n0 + l / 32];
        const float bv = s_h[(32 * op + l % 32) * CP + n0 + l / 32];
        inter = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, inter, 0, 0, 0);
    }

    // epilogue: y = intra + e^{a c_t} (C_t·h_in) + D x, times silu(z); lane l owns channel p and four runs
    // of four consecutive steps
    const int p = 32 * op + l % 32;
    const int64_t ch = h * kP + p;
    const float dsk = a.D ? a.D[ch] : 0.0f;
    const int64_t row = (ib * a.H * kP + ch) * a.L;
    const T *zg = static_cast<const T *>(a.z);
    T *yg = static_cast<T *>(a.y);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int t = 32 * ot + d_row(r, l);
        if (t0 + t >= a.L) continue;
        float v = acc[r] + exp2_fast(s_cum[t]) * inter[r] + dsk * s_x[p * kXP + t];
        if (zg) v *= silu(widen(zg[row + t0 + t]));
        yg[row + t0 + t] = narrow<T>(v);
    }
}

template <typename T, int N>
hipError_t launch_n(const SsdArgs &a, hipStream_t stream) {
    const unsigned chunks = (unsigned)(a.b * a.H * a.nc);
    hipLaunchKernelGGL((ssd_state_kernel<T, N>), dim3(chunks), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t elems = a.b * a.H * kP * N;
    hipLaunchKernelGGL((ssd_pass_kernel<N>), dim3((unsigned)((elems + 255) / 256)), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((ssd_out_kernel<T, N>), dim3(chunks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const SsdArgs &a, int64_t N, hipStream_t stream) {
    switch (N) {
        case 32: return launch_n<T, 32>(a, stream);
        case 64: return launch_n<T, 64>(a, stream);
        case 128: return launch_n<T, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int64_t ssd_scratch_floats(int64_t b, int64_t H, int64_t L, int64_t N) {
    const int64_t nc = (L + kQ - 1) / kQ;
    return b * H * nc * (kP * N + 1);
}

hipError_t launch_ssd(const SsdLaunch &p, hipStream_t stream) {
    if (p.L == 0) return hipSuccess;
    SsdArgs a{};
    a.x = p.x; a.delta = p.delta; a.B = p.B; a.C = p.C; a.z = p.z;
    a.A = p.A; a.D = p.D; a.h0 = p.h0; a.y = p.y; a.hT = p.hT;
    a.b = p.b; a.H = p.H; a.L = p.L;
    a.nc = (p.L + kQ - 1) / kQ;
    a.S = p.scratch;
    a.decay = p.scratch + a.b * a.H * a.nc * (kP * p.N);
    if (p.bf16) return launch_typed<uint16_t>(a, p.N, stream);
    return launch_typed<float>(a, p.N, stream);
}

}  // namespace ssm
