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
// N) and the chunk state X_w Bᵀ (P×N over Q). fp32 storage runs them on v_mfma_f32_32x32x2f32 (fp32 in,
// fp32 accumulate); bf16 storage on v_mfma_f32_32x32x16_bf16 (bf16 in, fp32 accumulate): inputs stored as
// bf16 enter exactly, and each fp32 operand (the decayed products, the weighted inputs, the entering state)
// enters as the sum of two bf16 numbers, hi = bf16(v) and lo = bf16(v − hi), in two products, which keeps
// about 16 bits of it. Chunk states and entering states pass through HBM as fp32 for both storage types
// (kept in bf16 they were measured to cost most of the bf16 tolerance).
//
// Three kernels:
//   ssd_state_kernel   per (b, h, chunk): the chunk's own state contribution S_c [P][N] and its decay.
//   ssd_pass_kernel    per (b, h, p, n): walks the chunks in order, replacing S_c by the state entering
//                      chunk c and writing the final state.
//   ssd_out_kernel     per (b, h, chunk): the outputs of the chunk from its inputs and entering state.
// Where b·H·N/64 workgroups fill the device, ssd_scan_kernel (ssd_scan.hip) takes the place of the first
// two: it walks each head's chunks in order with the state in its MFMA accumulators, so the chunk
// states never pass through HBM.
//
// MFMA lane layouts (checked on the device): 32x32x2 f32: lane l supplies A[l % 32][l / 32] and
// B[l / 32][l % 32]; 32x32x16 bf16: lane l supplies A[l % 32][8(l / 32) + e] and B[8(l / 32) + e][l % 32],
// e < 8; for both, result register r of lane l is D[8(r / 4) + 4(l / 32) + r % 4][l % 32].
#include "device_common.h"
#include "launch.h"
#include "ssd_common.h"

namespace ssm {
namespace {

using namespace ssd;

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

// Copy `rows` rows of `cols` elements (a multiple of 4) from global memory (row stride gstride, rows
// at and past row_limit read as zeros) into LDS rows of stride lstride, as fp32, with 4-element loads
// spread over the workgroup; each value is multiplied by scale[col] when scale is given.
template <typename T>
__device__ __forceinline__ void stage_rows(const T *g, int64_t gstride, int rows, int cols, int64_t row_limit,
                                           int64_t col_limit, bool vec, float *lds, int lstride,
                                           const float *scale = nullptr) {
    const int per_row = cols / 4;
    for (int idx = threadIdx.x; idx < rows * per_row; idx += kThreads) {
        const int r = idx / per_row, c4 = (idx % per_row) * 4;
        float4 v = r < row_limit ? load4<T>(g + r * gstride, c4, col_limit, vec) : make_float4(0.f, 0.f, 0.f, 0.f);
        if (scale) {
            v.x *= scale[c4]; v.y *= scale[c4 + 1]; v.z *= scale[c4 + 2]; v.w *= scale[c4 + 3];
        }
        *reinterpret_cast<float4 *>(lds + r * lstride + c4) = v;
    }
}

template <typename T, int N>
__global__ __launch_bounds__(kThreads) void ssd_state_kernel(SsdArgs a) {
    __shared__ float s_cum[kQ], s_beta[kQ];
    __shared__ __align__(16) float s_w[kQ];
    __shared__ __align__(16) float s_x[kP * kMS];  // x·w [p][s]
    __shared__ __align__(16) float s_bt[N * kMS];  // Bᵀ [n][s]
    const int64_t c = blockIdx.x % a.nc, bh = blockIdx.x / a.nc;
    const int64_t ib = bh / a.H, h = bh % a.H;
    const int64_t t0 = c * kQ;
    const float ah = a.A[h];
    chunk_scalars<T>(a, bh, t0, ah, s_cum, s_beta);
    {
        // Bᵀ: each thread reads 4 consecutive n of one step and writes them down a column
        const T *g = static_cast<const T *>(a.B) + (ib * a.L + t0) * N;
        for (int idx = threadIdx.x; idx < kQ * (N / 4); idx += kThreads) {
            const int t = idx / (N / 4), n4 = (idx % (N / 4)) * 4;
            const float4 v = t0 + t < a.L ? load4<T>(g + t * N, n4, N, a.vec_bc) : make_float4(0.f, 0.f, 0.f, 0.f);
            s_bt[(n4 + 0) * kMS + t] = v.x;
            s_bt[(n4 + 1) * kMS + t] = v.y;
            s_bt[(n4 + 2) * kMS + t] = v.z;
            s_bt[(n4 + 3) * kMS + t] = v.w;
        }
    }
    __syncthreads();
    if (threadIdx.x < kQ) {
        const float cend = s_cum[kQ - 1];
        s_w[threadIdx.x] = exp2_fast(cend - s_cum[threadIdx.x]) * s_beta[threadIdx.x];
        if (threadIdx.x == 0) a.decay[bh * a.nc + c] = exp2_fast(cend);
    }
    __syncthreads();
    stage_rows<T>(static_cast<const T *>(a.x) + ((ib * a.H + h) * kP) * a.L + t0, a.L, kP, kQ, kP, a.L - t0, a.vec,
                  s_x, kMS, s_w);
    __syncthreads();
    // S[p][n] = Σ_s x[p][s] w_s B[s][n]: 2 × N/32 tiles of 32×32 over the four wavefronts, K = 64 steps
    const int l = lane(), hi = l / 32;
    float *S = a.S + (bh * a.nc + c) * (int64_t)(kP * N);
    for (int tile = wave(); tile < 2 * (N / 32); tile += 4) {
        const int qp = tile % 2, qn = tile / 2;
        const float *xr = s_x + (32 * qp + l % 32) * kMS + 32 * hi;
        const float *br = s_bt + (32 * qn + l % 32) * kMS + 32 * hi;
        f16v acc = {};
        mfma_tile<32>(acc, [&](int j) { return *reinterpret_cast<const float4 *>(xr + j); },
                      [&](int j) { return *reinterpret_cast<const float4 *>(br + j); });
#pragma unroll
        for (int r = 0; r < 16; ++r) S[(32 * qp + d_row(r, l)) * N + 32 * qn + l % 32] = acc[r];
    }
}

// One thread per (b, h, p, n): h ← decay_c·h + S_c over the chunks, leaving in S_c the state that enters
// chunk c; the last value is the final state. The chunk states are read eight chunks ahead (they do not
// depend on h), so the chain waits on one round of loads per eight chunks. SS is the storage type of the
// chunk states (fp32 here).
template <typename SS, int N>
__global__ __launch_bounds__(256) void ssd_pass_kernel(SsdArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= a.b * a.H * kP * N) return;
    const int64_t pn = gid % (kP * N), bh = gid / (kP * N);
    float hv = a.h0 ? a.h0[bh * (kP * N) + pn] : 0.0f;  // [b][H·P][N] = [b·H][P·N]
    SS *S = reinterpret_cast<SS *>(a.S) + bh * a.nc * (kP * N) + pn;
    const float *dec = a.decay + bh * a.nc;
    constexpr int U = 8;
    for (int64_t c0 = 0; c0 < a.nc; c0 += U) {
        float sv[U], dv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool in = c0 + u < a.nc;
            sv[u] = in ? widen(S[(c0 + u) * (kP * N)]) : 0.0f;
            dv[u] = in ? dec[c0 + u] : 1.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c0 + u < a.nc) S[(c0 + u) * (kP * N)] = narrow<SS>(hv);
            hv = __builtin_fmaf(dv[u], hv, sv[u]);
        }
    }
    if (a.hT) a.hT[bh * (kP * N) + pn] = hv;
}

template <typename T, int N>
__global__ __launch_bounds__(kThreads) void ssd_out_kernel(SsdArgs a) {
    constexpr int NS = N + 4;                                   // LDS row stride of N-wide rows
    constexpr int BM = (kQ * NS > kQ * kMS) ? kQ * NS : kQ * kMS;
    __shared__ float s_cum[kQ], s_beta[kQ];
    __shared__ __align__(16) float s_c[BM];       // C [t][n]; at the end the outputs [p][t]
    __shared__ __align__(16) float s_bm[BM];      // B [s][n], then the decayed products M [t][s]
    __shared__ __align__(16) float s_x[kP * kMS]; // x [p][s]
    const int64_t c = blockIdx.x % a.nc, bh = blockIdx.x / a.nc;
    const int64_t ib = bh / a.H, h = bh % a.H;
    const int64_t t0 = c * kQ;
    const float ah = a.A[h];
    const int l = lane(), w = wave(), hi = l / 32;
    constexpr int HN = N / 2;
    const int ot = w / 2, op = w % 2;  // this wavefront's output tile: rows t in [32·ot, +32), channels [32·op, +32)
    // the entering-state operand of the C·h_inᵀ product (row p = 32·op + l % 32, n = hi·N/2 ..) goes
    // straight to registers, its loads issued first so that they overlap the staging below
    float4 hv[HN / 4];
    {
        const float *hr = a.S + (bh * a.nc + c) * (int64_t)(kP * N) + (32 * op + l % 32) * N + hi * HN;
#pragma unroll
        for (int j = 0; j < HN / 4; ++j) hv[j] = *reinterpret_cast<const float4 *>(hr + 4 * j);
    }
    chunk_scalars<T>(a, bh, t0, ah, s_cum, s_beta);
    const T *xg = static_cast<const T *>(a.x) + ((ib * a.H + h) * kP) * a.L + t0;  // row p at + p·L
    stage_rows<T>(static_cast<const T *>(a.C) + (ib * a.L + t0) * N, N, kQ, N, a.L - t0, N, a.vec_bc, s_c, NS);
    stage_rows<T>(static_cast<const T *>(a.B) + (ib * a.L + t0) * N, N, kQ, N, a.L - t0, N, a.vec_bc, s_bm, NS);
    stage_rows<T>(xg, a.L, kP, kQ, kP, a.L - t0, a.vec, s_x, kMS);
    __syncthreads();

    // G = C Bᵀ on the tiles at or below the diagonal (wavefronts 0..2), then M = G ∘ e^{a(c_t − c_s)} β_s
    // for s <= t; wavefront 3 clears the tile above the diagonal.
    f16v g = {};
    const int qt = w == 0 ? 0 : 1, qs = w == 2 ? 1 : 0;
    if (w < 3) {
        const float *cr = s_c + (32 * qt + l % 32) * NS + hi * HN;
        const float *br = s_bm + (32 * qs + l % 32) * NS + hi * HN;
        mfma_tile<HN>(g, [&](int j) { return *reinterpret_cast<const float4 *>(cr + j); },
                      [&](int j) { return *reinterpret_cast<const float4 *>(br + j); });
    }
    __syncthreads();  // B is no longer read: its space takes M
    if (w < 3) {
        const int s = 32 * qs + l % 32;
        const float cs = s_cum[s], bs = s_beta[s];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = 32 * qt + d_row(r, l);
            s_bm[t * kMS + s] = s <= t ? g[r] * exp2_fast(s_cum[t] - cs) * bs : 0.0f;
        }
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s_bm[d_row(r, l) * kMS + 32 + l % 32] = 0.0f;
    }
    __syncthreads();

    f16v acc = {}, inter = {};
    {
        const float *mr = s_bm + (32 * ot + l % 32) * kMS + 32 * hi;
        const float *xr = s_x + (32 * op + l % 32) * kMS + 32 * hi;
        mfma_tile<32>(acc, [&](int j) { return *reinterpret_cast<const float4 *>(mr + j); },
                      [&](int j) { return *reinterpret_cast<const float4 *>(xr + j); });
        const float *cr = s_c + (32 * ot + l % 32) * NS + hi * HN;
        mfma_tile<HN>(inter, [&](int j) { return *reinterpret_cast<const float4 *>(cr + j); },
                      [&](int j) { return hv[j / 4]; });
    }
    __syncthreads();  // C is no longer read: its space takes the outputs [p][t]
    {
        const int p = 32 * op + l % 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = 32 * ot + d_row(r, l);
            s_c[p * kMS + t] = acc[r] + exp2_fast(s_cum[t]) * inter[r];
        }
    }
    __syncthreads();
    // y = (that) + D x, times silu(z), written row by row in 4-step pieces
    const T *zg = static_cast<const T *>(a.z);
    T *yg = static_cast<T *>(a.y);
    const int64_t lim = a.L - t0;
    for (int idx = threadIdx.x; idx < kP * (kQ / 4); idx += kThreads) {
        const int p = idx / (kQ / 4), t4 = (idx % (kQ / 4)) * 4;
        if (t4 >= lim) continue;
        const int64_t ch = h * kP + p;
        const int64_t off = (ib * a.H * kP + ch) * a.L + t0 + t4;
        const float dsk = a.D ? a.D[ch] : 0.0f;
        const float4 o = *reinterpret_cast<const float4 *>(s_c + p * kMS + t4);
        const float4 xv = *reinterpret_cast<const float4 *>(s_x + p * kMS + t4);
        float v[4] = {o.x + dsk * xv.x, o.y + dsk * xv.y, o.z + dsk * xv.z, o.w + dsk * xv.w};
        if (zg) {
            const float4 zv = load4<T>(zg + off - t4, t4, lim, a.vec);
            v[0] *= silu(zv.x); v[1] *= silu(zv.y); v[2] *= silu(zv.z); v[3] *= silu(zv.w);
        }
        if (a.vec && t4 + 4 <= lim) {
            if constexpr (sizeof(T) == 4) {
                *reinterpret_cast<float4 *>(yg + off) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
                uint2 pk;
                pk.x = (uint32_t)narrow<T>(v[0]) | ((uint32_t)narrow<T>(v[1]) << 16);
                pk.y = (uint32_t)narrow<T>(v[2]) | ((uint32_t)narrow<T>(v[3]) << 16);
                *reinterpret_cast<uint2 *>(yg + off) = pk;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (t4 + e < lim) yg[off + e] = narrow<T>(v[e]);
        }
    }
}

// ---- bf16 storage: the same three steps on the bf16 MFMA -------------------------------------------

// Copy rows of `cols` bf16 elements (a multiple of 8) into LDS rows of stride lstride, 16 bytes at a time;
// rows at and past row_limit and columns at and past col_limit read as zeros.
__device__ __forceinline__ void stage_rows_bf16(const uint16_t *g, int64_t gstride, int rows, int cols,
                                                int64_t row_limit, int64_t col_limit, bool vec, uint16_t *lds,
                                                int lstride) {
    const int per_row = cols / 8;
    for (int idx = threadIdx.x; idx < rows * per_row; idx += kThreads) {
        const int r = idx / per_row, c8 = (idx % per_row) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < row_limit) {
            const uint16_t *src = g + r * gstride + c8;
            if (vec && c8 + 8 <= col_limit) {
                v = *reinterpret_cast<const uint4 *>(src);
            } else {
                uint16_t e[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) e[k] = c8 + k < col_limit ? src[k] : (uint16_t)0;
                __builtin_memcpy(&v, e, sizeof(v));
            }
        }
        *reinterpret_cast<uint4 *>(lds + r * lstride + c8) = v;
    }
}

template <int N>
__global__ __launch_bounds__(kThreads) void ssd_state_kernel_bf16(SsdArgs a) {
    __shared__ float s_cum[kQ], s_beta[kQ], s_w[kQ];
    __shared__ __align__(16) float s_x[kP * kMS];     // x·w [p][s], fp32
    __shared__ __align__(16) uint16_t s_bt[N * kMH];  // Bᵀ [n][s]
    const int64_t c = blockIdx.x % a.nc, bh = blockIdx.x / a.nc;
    const int64_t ib = bh / a.H, h = bh % a.H;
    const int64_t t0 = c * kQ;
    const float ah = a.A[h];
    chunk_scalars<uint16_t>(a, bh, t0, ah, s_cum, s_beta);
    {
        const uint16_t *g = static_cast<const uint16_t *>(a.B) + (ib * a.L + t0) * N;
        for (int idx = threadIdx.x; idx < kQ * N; idx += kThreads) {
            const int t = idx / N, n = idx % N;
            s_bt[n * kMH + t] = t0 + t < a.L ? g[idx] : (uint16_t)0;
        }
    }
    __syncthreads();
    if (threadIdx.x < kQ) {
        const float cend = s_cum[kQ - 1];
        s_w[threadIdx.x] = exp2_fast(cend - s_cum[threadIdx.x]) * s_beta[threadIdx.x];
        if (threadIdx.x == 0) a.decay[bh * a.nc + c] = exp2_fast(cend);
    }
    __syncthreads();
    {
        const uint16_t *xg = static_cast<const uint16_t *>(a.x) + ((ib * a.H + h) * kP) * a.L + t0;
        for (int idx = threadIdx.x; idx < kP * (kQ / 4); idx += kThreads) {
            const int p = idx / (kQ / 4), s4 = (idx % (kQ / 4)) * 4;
            const float4 v = load4<uint16_t>(xg + p * a.L, s4, a.L - t0, a.vec);
            *reinterpret_cast<float4 *>(s_x + p * kMS + s4) =
                make_float4(v.x * s_w[s4], v.y * s_w[s4 + 1], v.z * s_w[s4 + 2], v.w * s_w[s4 + 3]);
        }
    }
    __syncthreads();
    const int l = lane(), hi = l / 32;
    float *S = a.S + (bh * a.nc + c) * (int64_t)(kP * N);
    for (int tile = wave(); tile < 2 * (N / 32); tile += 4) {
        const int qp = tile % 2, qn = tile / 2;
        f16v acc = {};
        mfma_tile_split<32, true>(acc, s_x + (32 * qp + l % 32) * kMS + 32 * hi,
                                  s_bt + (32 * qn + l % 32) * kMH + 32 * hi);
#pragma unroll
        for (int r = 0; r < 16; ++r) S[(32 * qp + d_row(r, l)) * N + 32 * qn + l % 32] = acc[r];
    }
}

template <int N>
__global__ __launch_bounds__(kThreads) void ssd_out_kernel_bf16(SsdArgs a) {
    constexpr int NH = N + 8;                                   // LDS row stride (bf16) of N-wide rows
    constexpr int OUTF = kP * kMS;                              // fp32 [64][kMS] (M, then the outputs)
    constexpr int CB = (kQ * NH > OUTF * 2) ? kQ * NH : OUTF * 2;  // bf16 units
    __shared__ float s_cum[kQ], s_beta[kQ];
    __shared__ __align__(16) uint16_t s_c[CB];        // C [t][n]; at the end the outputs [p][t] (fp32)
    __shared__ __align__(16) uint16_t s_bm[CB];       // B [s][n], then M [t][s] (fp32)
    __shared__ __align__(16) uint16_t s_x[kP * kMH];  // x [p][s]
    const int64_t c = blockIdx.x % a.nc, bh = blockIdx.x / a.nc;
    const int64_t ib = bh / a.H, h = bh % a.H;
    const int64_t t0 = c * kQ;
    const float ah = a.A[h];
    const int l = lane(), w = wave(), hi = l / 32;
    constexpr int HN = N / 2;
    const int ot = w / 2, op = w % 2;  // this wavefront's output tile
    // the entering-state operand (row p = 32·op + l % 32, n = hi·N/2 ..) straight to registers, first
    float4 hv[HN / 4];
    {
        const float *hr = a.S + (bh * a.nc + c) * (int64_t)(kP * N) + (32 * op + l % 32) * N + hi * HN;
#pragma unroll
        for (int j = 0; j < HN / 4; ++j) hv[j] = *reinterpret_cast<const float4 *>(hr + 4 * j);
    }
    chunk_scalars<uint16_t>(a, bh, t0, ah, s_cum, s_beta);
    const uint16_t *xg = static_cast<const uint16_t *>(a.x) + ((ib * a.H + h) * kP) * a.L + t0;
    stage_rows_bf16(static_cast<const uint16_t *>(a.C) + (ib * a.L + t0) * N, N, kQ, N, a.L - t0, N, a.vec_bc, s_c, NH);
    stage_rows_bf16(static_cast<const uint16_t *>(a.B) + (ib * a.L + t0) * N, N, kQ, N, a.L - t0, N, a.vec_bc, s_bm, NH);
    stage_rows_bf16(xg, a.L, kP, kQ, kP, a.L - t0, a.vec8, s_x, kMH);
    __syncthreads();

    f16v g = {};
    const int qt = w == 0 ? 0 : 1, qs = w == 2 ? 1 : 0;
    if (w < 3) mfma_tile_bf16<HN>(g, s_c + (32 * qt + l % 32) * NH + hi * HN, s_bm + (32 * qs + l % 32) * NH + hi * HN);
    __syncthreads();  // B is no longer read: its space takes M (fp32)
    float *s_m = reinterpret_cast<float *>(s_bm);
    if (w < 3) {
        const int s = 32 * qs + l % 32;
        const float cs = s_cum[s], bs = s_beta[s];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = 32 * qt + d_row(r, l);
            s_m[t * kMS + s] = s <= t ? g[r] * exp2_fast(s_cum[t] - cs) * bs : 0.0f;
        }
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s_m[d_row(r, l) * kMS + 32 + l % 32] = 0.0f;
    }
    __syncthreads();

    f16v acc = {}, inter = {};
    mfma_tile_split<32, true>(acc, s_m + (32 * ot + l % 32) * kMS + 32 * hi, s_x + (32 * op + l % 32) * kMH + 32 * hi);
    {
        // the entering state (fp32) enters as hi + lo
        const uint16_t *cr = s_c + (32 * ot + l % 32) * NH + hi * HN;
#pragma unroll
        for (int j = 0; j < HN / 8; ++j) {
            bf8v h8, l8;
            split8(hv[2 * j], hv[2 * j + 1], h8, l8);
            const bf8v c8 = *reinterpret_cast<const bf8v *>(cr + 8 * j);
            inter = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c8, h8, inter, 0, 0, 0);
            inter = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c8, l8, inter, 0, 0, 0);
        }
    }
    __syncthreads();  // C is no longer read: its space takes the outputs
    float *s_o = reinterpret_cast<float *>(s_c);
    {
        const int p = 32 * op + l % 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = 32 * ot + d_row(r, l);
            s_o[p * kMS + t] = acc[r] + exp2_fast(s_cum[t]) * inter[r];
        }
    }
    __syncthreads();
    const uint16_t *zg = static_cast<const uint16_t *>(a.z);
    uint16_t *yg = static_cast<uint16_t *>(a.y);
    const int64_t lim = a.L - t0;
    for (int idx = threadIdx.x; idx < kP * (kQ / 4); idx += kThreads) {
        const int p = idx / (kQ / 4), t4 = (idx % (kQ / 4)) * 4;
        if (t4 >= lim) continue;
        const int64_t ch = h * kP + p;
        const int64_t off = (ib * a.H * kP + ch) * a.L + t0 + t4;
        const float dsk = a.D ? a.D[ch] : 0.0f;
        const float4 o = *reinterpret_cast<const float4 *>(s_o + p * kMS + t4);
        const uint16_t *xs = s_x + p * kMH + t4;
        float v[4] = {o.x + dsk * widen(xs[0]), o.y + dsk * widen(xs[1]), o.z + dsk * widen(xs[2]),
                      o.w + dsk * widen(xs[3])};
        if (zg) {
            const float4 zv = load4<uint16_t>(zg + off - t4, t4, lim, a.vec);
            v[0] *= silu(zv.x); v[1] *= silu(zv.y); v[2] *= silu(zv.z); v[3] *= silu(zv.w);
        }
        if (a.vec && t4 + 4 <= lim) {
            uint2 pk;
            pk.x = (uint32_t)narrow<uint16_t>(v[0]) | ((uint32_t)narrow<uint16_t>(v[1]) << 16);
            pk.y = (uint32_t)narrow<uint16_t>(v[2]) | ((uint32_t)narrow<uint16_t>(v[3]) << 16);
            *reinterpret_cast<uint2 *>(yg + off) = pk;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (t4 + e < lim) yg[off + e] = narrow<uint16_t>(v[e]);
        }
    }
}

template <typename T, int N>
hipError_t launch_n(const SsdArgs &a, hipStream_t stream) {
    const unsigned chunks = (unsigned)(a.b * a.H * a.nc);
    if constexpr (sizeof(T) == 2 && N % 64 == 0) {
        if (a.fused_all) return launch_fused(a, N, stream);
    }
    if constexpr (N % 64 == 0) {
        if (a.fused) {
            hipError_t e = launch_state_walk(a, N, sizeof(T) == 2, stream);
            if (e != hipSuccess) return e;
            if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((ssd_out_kernel_bf16<N>), dim3(chunks), dim3(kThreads), 0, stream, a);
            else hipLaunchKernelGGL((ssd_out_kernel<T, N>), dim3(chunks), dim3(kThreads), 0, stream, a);
            return hipGetLastError();
        }
    }
    if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((ssd_state_kernel_bf16<N>), dim3(chunks), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((ssd_state_kernel<T, N>), dim3(chunks), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t elems = a.b * a.H * kP * N;
    hipLaunchKernelGGL((ssd_pass_kernel<float, N>), dim3((unsigned)((elems + 255) / 256)), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((ssd_out_kernel_bf16<N>), dim3(chunks), dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((ssd_out_kernel<T, N>), dim3(chunks), dim3(kThreads), 0, stream, a);
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

bool ssd_single_walk(int64_t b, int64_t H, int64_t N, bool bf16, int cus) {
    return bf16 && (N == 64 || N == 128) && b * H >= 2 * (int64_t)cus;
}

int64_t ssd_scratch_floats(int64_t b, int64_t H, int64_t L, int64_t N, bool bf16, int cus) {
    if (ssd_single_walk(b, H, N, bf16, cus)) return 0;
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
    const int64_t es = p.bf16 ? 2 : 4;
    auto aligned = [&](const void *q) { return (reinterpret_cast<uintptr_t>(q) & (uintptr_t)(4 * es - 1)) == 0; };
    a.vec = (p.L % 4) == 0 && aligned(p.x) && aligned(p.y) && (!p.z || aligned(p.z));
    a.vec_bc = aligned(p.B) && aligned(p.C);  // N is a multiple of 32
    a.vec8 = p.bf16 && (p.L % 8) == 0 && (reinterpret_cast<uintptr_t>(p.x) & 15) == 0;
    a.decay = p.scratch ? p.scratch + a.b * a.H * a.nc * (kP * p.N) : nullptr;
    // the fused state walk runs b·H·N/64 workgroups of four wavefronts; it pays once they give every
    // compute unit two
    a.fused = p.N % 64 == 0 && a.b * a.H * (p.N / 64) >= 2 * (int64_t)p.cus;
    a.vec_bc16 = ((reinterpret_cast<uintptr_t>(p.B) | reinterpret_cast<uintptr_t>(p.C)) & 15) == 0;
    // bf16 storage with b·H >= 2 workgroups per CU: the whole form in one walk per (b, head)
    a.fused_all = ssd_single_walk(a.b, a.H, p.N, p.bf16, p.cus);
    if (p.bf16) return launch_typed<uint16_t>(a, p.N, stream);
    return launch_typed<float>(a, p.N, stream);
}

}  // namespace ssm
