// ssd_scan.hip — the chunk states of the scalar-decay chunked form and their pass in one kernel.
//
// Page "State Space Models（SSM）とMamba" §4.6 (state space duality) with the unrolled recurrence of page
// "Mambaとは？Transformer以外の系列モデル", section Mambaの核心は入力依存のDelta、B、C: with A = a·I the
// state leaving a chunk of Q steps is h_out = e^{a c_end} h_in + Σ_s e^{a(c_end − c_s)} β_s B_s x_sᵀ
// (c the in-chunk running sum of Δ, β the ZOH input coefficient), a dense product per chunk.
#include <type_traits>

#include "launch.h"
#include "ssd_common.h"

namespace ssm {
namespace ssd {
namespace {

// ---- chunk states and their pass fused: one workgroup walks the chunks of (b, h) in order ------------
//
// Workgroup (b, h, nb) keeps the columns n0 .. n0+63 (n0 = 64·nb) of the head's [P][N] state in its
// MFMA accumulators (wavefront w: rows 32(w % 2) .., columns n0 + 32(w / 2) ..) and for each chunk c
// writes them out as the state entering c, then takes h ← e^{a c_end} h + X_w Bᵀ with the chunk's
// weighted inputs X_w[p][s] = x[p][s]·e^{a(c_end − c_s)} β_s. That replaces the chunk states' round
// trip through HBM and the separate pass over them. It needs b·H·N/64 workgroups to fill the device, so
// the three-kernel form serves the shapes with fewer.

// Workgroup barrier ordering LDS only: global loads and stores stay in flight across it (the next
// chunk's operands arrive while this one is multiplied, and the entering states drain meanwhile).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 64 lanes of a wavefront: DPP row shifts within each row of 16 lanes
// (lanes shifted in from outside the row add 0), then each row adds the totals of the rows before it,
// read with readlane.
__device__ __forceinline__ float wave_prefix_sum(float v) {
    auto shr = [](float x, auto k) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + decltype(k)::value, 0xf, 0xf, false));
    };
    v += shr(v, std::integral_constant<int, 1>{});
    v += shr(v, std::integral_constant<int, 2>{});
    v += shr(v, std::integral_constant<int, 4>{});
    v += shr(v, std::integral_constant<int, 8>{});
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47));
    const int row = (threadIdx.x & 63) >> 4;
    const float before = row == 0 ? 0.0f : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2;
    return v + before;
}

// Four consecutive elements row[i .. i+3] in storage form (fp32: float4, bf16: the 8 bytes as uint2),
// zeros at and past `limit`.
template <typename T>
__device__ __forceinline__ typename std::conditional<sizeof(T) == 2, uint2, float4>::type raw4(
    const T *row, int64_t i, int64_t limit, bool vec) {
    if constexpr (sizeof(T) == 4) {
        return load4<T>(row, i, limit, vec);
    } else {
        if (vec && i + 4 <= limit) return *reinterpret_cast<const uint2 *>(row + i);
        uint16_t e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) e[k] = i + k < limit ? row[i + k] : (uint16_t)0;
        uint2 r;
        __builtin_memcpy(&r, e, sizeof(r));
        return r;
    }
}
__device__ __forceinline__ void raw_elems(const float4 &v, float (&o)[4]) { o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w; }
__device__ __forceinline__ void raw_elems(const uint2 &v, float (&o)[4]) {
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
}
__device__ __forceinline__ void raw_bits(const uint2 &v, uint16_t (&o)[4]) {
    o[0] = (uint16_t)(v.x & 0xffffu); o[1] = (uint16_t)(v.x >> 16); o[2] = (uint16_t)(v.y & 0xffffu); o[3] = (uint16_t)(v.y >> 16);
}

// As mfma_tile_split<W, true> with the fp32 operand row scaled elementwise by wrow (same k) on the way in.
template <int W>
__device__ __forceinline__ void mfma_tile_split_scaled(f16v &acc, const float *frow, const float *wrow,
                                                       const uint16_t *brow) {
#pragma unroll
    for (int j = 0; j < W / 8; ++j) {
        float4 u = *reinterpret_cast<const float4 *>(frow + 8 * j), v = *reinterpret_cast<const float4 *>(frow + 8 * j + 4);
        const float4 wu = *reinterpret_cast<const float4 *>(wrow + 8 * j), wv = *reinterpret_cast<const float4 *>(wrow + 8 * j + 4);
        u.x *= wu.x; u.y *= wu.y; u.z *= wu.z; u.w *= wu.w;
        v.x *= wv.x; v.y *= wv.y; v.z *= wv.z; v.w *= wv.w;
        bf8v h8, l8;
        split8(u, v, h8, l8);
        const bf8v o8 = *reinterpret_cast<const bf8v *>(brow + 8 * j);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h8, o8, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l8, o8, acc, 0, 0, 0);
    }
}

template <typename T, int N>
__global__ __launch_bounds__(kThreads) void ssd_scan_kernel(SsdArgs a) {
    static_assert(N % 64 == 0, "64 state columns per workgroup");
    constexpr bool BF = sizeof(T) == 2;
    constexpr int NB = N / 64;
    constexpr int BS = BF ? kMH : kMS;  // LDS row stride of the Bᵀ rows
    typedef typename std::conditional<BF, uint16_t, float>::type BT;
    typedef typename std::conditional<BF, uint2, float4>::type Raw;
    __shared__ __align__(16) float s_w[4 * kQ];     // each wavefront's copy of the chunk weights
    __shared__ __align__(16) float s_x[kP * kMS];  // x [p][s] (fp32)
    __shared__ __align__(16) BT s_bt[64 * BS];      // Bᵀ [n − n0][s] (storage type)
    const int64_t nb = blockIdx.x % NB, bh = blockIdx.x / NB;
    const int64_t ib = bh / a.H, h = bh % a.H;
    const int n0 = 64 * (int)nb;
    const float ah = a.A[h];
    const int l = lane(), w = wave(), hi = l / 32;
    const int qp = w % 2, qn = w / 2;
    const int tid = threadIdx.x;
    // this lane's elements of the state tile: acc[r] = h[32 qp + d_row(r, l)][n0 + 32 qn + l % 32]
    auto st_off = [&](int r) { return (int64_t)(32 * qp + d_row(r, l)) * N + n0 + 32 * qn + l % 32; };
    f16v acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = a.h0 ? a.h0[bh * (kP * N) + st_off(r)] : 0.0f;

    const T *dg = static_cast<const T *>(a.delta) + bh * a.L;
    const T *bg = static_cast<const T *>(a.B) + ib * a.L * N + n0;
    const T *xg = static_cast<const T *>(a.x) + ((ib * a.H + h) * kP) * a.L;
    // the chunk's operands in registers: Δ of step l (every wavefront), and for k < 4 four B values
    // (step br_, columns bq_ ..: 4 lanes per step, so that the transposed LDS stores below spread over
    // the banks) and four x values (channel xr_, steps xq_ ..: 16 lanes per channel row)
    auto br_ = [&](int) { return 16 * w + l / 4; };
    auto bq_ = [&](int k) { return 16 * k + 4 * (l % 4); };
    auto xr_ = [&](int k) { return (tid + k * kThreads) / 16; };
    auto xq_ = [&](int k) { return ((tid + k * kThreads) % 16) * 4; };
    float dtr = 0.0f;
    Raw bq[4], xq[4];
    auto load_chunk = [&](int64_t c) {
        const int64_t t0 = c * kQ;
        dtr = t0 + l < a.L ? widen(dg[t0 + l]) : 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = br_(k);
            bq[k] = raw4<T>(bg + (t0 + r) * N, bq_(k), t0 + r < a.L ? 64 : 0, a.vec_bc);
            xq[k] = raw4<T>(xg + xr_(k) * a.L + t0, xq_(k), a.L - t0, a.vec);
        }
    };
    load_chunk(0);
    for (int64_t c = 0; c < a.nc; ++c) {
        // every wavefront: the in-chunk running sum of Δ·a·log2 e, the ZOH coefficient, the weights
        // e^{a(c_end − c_s)} β_s (into its own LDS copy) and the chunk decay e^{a c_end}
        float dec;
        {
            const float u = dtr * (ah * kLog2e);
            const float abar = exp2_fast(u);
            const float beta = zoh_input_coef_log2(dtr, u, abar, 1.0f / ah);
            const float cu = wave_prefix_sum(u);
            const float cend = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cu), 63));
            s_w[kQ * w + l] = exp2_fast(cend - cu) * beta;
            dec = exp2_fast(cend);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = br_(k), q4 = bq_(k);
            if constexpr (BF) {
                uint16_t e[4];
                raw_bits(bq[k], e);
#pragma unroll
                for (int i = 0; i < 4; ++i) s_bt[(q4 + i) * BS + r] = e[i];
            } else {
                float e[4];
                raw_elems(bq[k], e);
#pragma unroll
                for (int i = 0; i < 4; ++i) s_bt[(q4 + i) * BS + r] = e[i];
            }
            float xv[4];
            raw_elems(xq[k], xv);
            *reinterpret_cast<float4 *>(s_x + xr_(k) * kMS + xq_(k)) = make_float4(xv[0], xv[1], xv[2], xv[3]);
        }
        if (c + 1 < a.nc) load_chunk(c + 1);
        lds_barrier();  // x and Bᵀ
        float *S = a.S + (bh * a.nc + c) * (int64_t)(kP * N);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            S[st_off(r)] = acc[r];
            acc[r] *= dec;
        }
        const float *xr = s_x + (32 * qp + l % 32) * kMS + 32 * hi;
        const float *wr = s_w + kQ * w + 32 * hi;
        const BT *br = s_bt + (32 * qn + l % 32) * BS + 32 * hi;
        if constexpr (BF) {
            mfma_tile_split_scaled<32>(acc, xr, wr, br);
        } else {
            mfma_tile<32>(acc,
                          [&](int j) {
                              const float4 xv = *reinterpret_cast<const float4 *>(xr + j);
                              const float4 wv = *reinterpret_cast<const float4 *>(wr + j);
                              return make_float4(xv.x * wv.x, xv.y * wv.y, xv.z * wv.z, xv.w * wv.w);
                          },
                          [&](int j) { return *reinterpret_cast<const float4 *>(br + j); });
        }
        lds_barrier();  // the next chunk's staging overwrites the LDS operands
    }
    if (a.hT) {
#pragma unroll
        for (int r = 0; r < 16; ++r) a.hT[bh * (kP * N) + st_off(r)] = acc[r];
    }
}

// ---- the whole chunked form in one ordered walk (bf16 storage) ---------------------------------------
//
// Workgroup (b, h) walks the chunks of one head in order and keeps its state in MFMA accumulators, so
// neither chunk states nor entering states touch HBM: it reads x, z, Δ, B, C once and writes y once.
// Per chunk (Q = 64 steps), with M[t][s] = (C_t·B_s) e^{a(c_t − c_s)} β_s for s <= t:
//   y_t = e^{a c_t} C_t·h_in + Σ_s M[t][s] x_s + D x_t, times silu(z);
//   h ← e^{a c_end} h + Σ_s e^{a(c_end − c_s)} β_s x_s B_sᵀ.
// Wavefront w owns the output tile of steps 32·T .. and channels 32·Pt .. (T = w & 1, Pt = w >> 1) and
// holds half of the state columns of its 32 channels, Hᵀ[n][p] for n in N/2 · T .. N/2 · T + N/2 − 1, as
// N/64 accumulator tiles; its partner w ^ 1 holds the other half. Each forms C·Hᵀ over its half for both
// step tiles and hands the partner the partial sum of the partner's tile through LDS.
//
// The accumulator layout does the transposes. Lane l of a 32×32 accumulator holds column l % 32 and,
// in registers 8κ .. 8κ+7, rows 16κ + {0..3, 8..11} + 4·(l / 32). Read as an MFMA operand those registers
// are the lane's eight k values of the K block 16κ .. 16κ+15 in that order, so a tile of Hᵀ[n][p] is
// directly the k = n operand of C·Hᵀ, and a tile of Mᵀ[s][t] (formed as B·Cᵀ) is the k = s operand of
// M·x. The other operand of each of those products (C and x rows in LDS) is read in the same k order:
// two 8-byte LDS reads per lane and K block; the state update's Bᵀ operand is read down the columns of
// B's rows, 2 bytes at a time. The decayed product tiles cross wavefronts as bf16 hi and lo planes in LDS
// in lane order, the partial sums of C·Hᵀ as fp32 in lane order.
//
// LDS holds the chunk's C, B and x (bf16), the decayed product tiles, the partial sums and the chunk's
// scalars, about 73 KB at N = 128, so two workgroups share a compute unit and each one's barriers and
// exponentials overlap the other's products. Two barriers per chunk: the second lets the next chunk's
// staging overwrite the operands while this chunk's outputs are formed from registers, the product
// tiles and the partial sums.
// AM (access mode): 0 element by element with a bound per element; 1 every row piece whole and aligned
// (L a multiple of 8; x, y, z, B, C aligned), loads and stores by 16 (8) bytes with one guard per piece;
// 2 as 1 with every chunk whole (L a multiple of 64, 64·L < 2^31): no guards, and each access is a base
// that is uniform over the workgroup plus a per-lane 32-bit offset kept across the walk.
template <int N, int AM>
__global__ __launch_bounds__(kThreads, AM > 0 ? 2 : 1) void ssd_fused_kernel(SsdArgs a) {
    constexpr bool VEC = AM > 0;
    static_assert(N == 64 || N == 128, "state widths");
    constexpr int NH = N + 8;       // bf16 row stride of N-wide LDS rows
    constexpr int HN = N / 2;
    constexpr int NS = N / 64;      // state tiles per wavefront
    constexpr int CK = N / 32;      // 16-byte pieces of C (and of B) per thread per chunk
    __shared__ __align__(16) float s_cum[kQ], s_beta[kQ], s_w[kQ], s_et[kQ];
    __shared__ __align__(16) uint16_t s_c[kQ * NH];    // C [t][n]
    __shared__ __align__(16) uint16_t s_b[kQ * NH];    // B [s][n]
    __shared__ __align__(16) uint16_t s_x[kP * kMH];   // x [p][s]
    __shared__ __align__(16) uint4 s_m[3 * 4 * kWave]; // decayed product tiles: [tile][K block, hi / lo][lane]
    __shared__ __align__(16) float4 s_i[4 * 4 * kWave]; // partial C·Hᵀ for the partner: [wavefront][4 registers][lane]
    const int64_t bh = blockIdx.x, ib = bh / a.H, h = bh % a.H;
    const float ah = a.A[h];
    const int l = lane(), w = wave(), hi = l / 32, lc = l % 32, tid = threadIdx.x;
    const int T = w & 1, Pt = w >> 1;
    const int p = 32 * Pt + lc;              // this lane's channel in the output and state tiles
    const int n0 = (N / 2) * T;              // the first state row this wavefront holds
    // the decayed product tiles Mᵀ[s][t] with s <= t: (S, T) = (0, 0), (0, 1), (1, 1), slot S + T,
    // formed by wavefronts 0, 1 and 3
    const bool gw = w != 2;
    const int gS = w == 3 ? 1 : 0;

    f16v acc[NS];  // acc[j][r] = h[p][n0 + 32 j + d_row(r, l)]
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[j][r] = a.h0 ? a.h0[bh * (kP * N) + (int64_t)p * N + n0 + 32 * j + d_row(r, l)] : 0.0f;

    const uint16_t *dg = static_cast<const uint16_t *>(a.delta) + bh * a.L;
    const uint16_t *cg = static_cast<const uint16_t *>(a.C) + ib * a.L * N;
    const uint16_t *bg = static_cast<const uint16_t *>(a.B) + ib * a.L * N;
    const uint16_t *xg = static_cast<const uint16_t *>(a.x) + ((ib * a.H + h) * kP) * a.L;
    const uint16_t *zg = a.z ? static_cast<const uint16_t *>(a.z) + ((ib * a.H + h) * kP + p) * a.L : nullptr;
    uint16_t *yg = static_cast<uint16_t *>(a.y) + ((ib * a.H + h) * kP + p) * a.L;
    // staging pieces: C row c_r(k) columns c_c(k) .. +7 (16 lanes per row); B row l, columns
    // 8(w + 4k) .. +7 (one row per lane); x row x_r(k), steps x_c(k) .. +7
    auto c_r = [&](int k, int t = threadIdx.x) { return (t + k * kThreads) / (N / 8); };
    auto c_c = [&](int k, int t = threadIdx.x) { return ((t + k * kThreads) % (N / 8)) * 8; };
    auto b_c = [&](int k) { return 8 * (w + 4 * k); };
    auto x_r = [&](int k, int t = threadIdx.x) { return (t + k * kThreads) / 8; };
    auto x_c = [&](int k, int t = threadIdx.x) { return ((t + k * kThreads) % 8) * 8; };
    // 8 consecutive bf16 of a row as raw bits, zeros at and past `limit`
    auto raw8 = [](const uint16_t *row, int64_t i, int64_t limit) {
        if (VEC) return i + 8 <= limit ? *reinterpret_cast<const uint4 *>(row + i) : make_uint4(0u, 0u, 0u, 0u);
        uint16_t e[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = i + k < limit ? row[i + k] : (uint16_t)0;
        uint4 r;
        __builtin_memcpy(&r, e, sizeof(r));
        return r;
    };
    const float dsk = a.D ? a.D[h * kP + p] : 0.0f;
    // AM 2: the per-lane offsets of the first piece of each access, in elements from the chunk's uniform
    // bases; piece k lies a fixed stride further (kThreads threads cover whole rows: C by kThreads/(N/8)
    // rows, B by 32 columns, x by 32 rows)
    const uint32_t coff = (uint32_t)(c_r(0) * N + c_c(0));
    const uint32_t boff = (uint32_t)(l * N + b_c(0));
    const uint32_t xoff = (uint32_t)(x_r(0) * a.L + x_c(0));
    const uint32_t poff = (uint32_t)(p * a.L + 32 * T + 4 * hi);  // z and y: channel p, steps 32 T + 4 hi ..
    const uint16_t *zh = a.z ? static_cast<const uint16_t *>(a.z) + (ib * a.H + h) * kP * a.L : nullptr;
    uint16_t *yh = static_cast<uint16_t *>(a.y) + (ib * a.H + h) * kP * a.L;

    uint16_t dtr = 0;  // Δ of step l of the chunk being loaded, raw (widened where it is used)
    float dec = 0.0f;
    // the chunk's operands in flight: vector values rather than arrays, so they always stay in registers
    // (an array can be left in scratch memory when registers run short)
    typedef uint32_t rawv __attribute__((ext_vector_type(4 * CK)));
    typedef uint32_t rawx __attribute__((ext_vector_type(8)));
    rawv cq, bq;
    rawx xq;
    auto put4 = [](auto &v, int k, const uint4 &q) {
        v[4 * k] = q.x; v[4 * k + 1] = q.y; v[4 * k + 2] = q.z; v[4 * k + 3] = q.w;
    };
    auto get4 = [](const auto &v, int k) { return make_uint4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]); };
    uint2 zq[4];
    // The loads take the thread index behind an empty asm, so that their per-lane addresses are formed at
    // each chunk rather than kept (and spilled) across the walk.
    auto load_chunk = [&](int64_t c) {
        if constexpr (AM == 2) {
            const int64_t t0 = c * kQ;
            const uint16_t *cb = cg + t0 * N, *bb = bg + t0 * N, *xb = xg + t0;
            dtr = dg[t0 + l];
#pragma unroll
            for (int k = 0; k < CK; ++k) {
                put4(cq, k, *reinterpret_cast<const uint4 *>(cb + k * (kThreads / (N / 8)) * N + coff));
                put4(bq, k, *reinterpret_cast<const uint4 *>(bb + 32 * k + boff));
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) put4(xq, k, *reinterpret_cast<const uint4 *>(xb + k * (kThreads / 8) * a.L + xoff));
            return;
        }
        int th = tid;
        asm volatile("" : "+v"(th));
        const int ln = th % kWave;
        const int64_t t0 = c * kQ;
        dtr = t0 + ln < a.L ? dg[t0 + ln] : (uint16_t)0;
#pragma unroll
        for (int k = 0; k < CK; ++k) {
            const int cr = c_r(k, th);
            put4(cq, k, raw8(cg + (t0 + cr) * N, c_c(k, th), t0 + cr < a.L ? N : 0));
            put4(bq, k, raw8(bg + (t0 + ln) * N, b_c(k), t0 + ln < a.L ? N : 0));
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) put4(xq, k, raw8(xg + x_r(k, th) * a.L + t0, x_c(k, th), a.L - t0));
    };
    // z at this lane's output positions: channel p, steps 32 T + 8q + 4 hi .. +3
    auto load_z = [&](int64_t c) {
        if constexpr (AM == 2) {
            if (zh) {
                const uint16_t *zb = zh + c * kQ;
#pragma unroll
                for (int q = 0; q < 4; ++q) zq[q] = *reinterpret_cast<const uint2 *>(zb + poff + 8 * q);
            }
            return;
        }
        int ln = l;
        asm volatile("" : "+v"(ln));
        const int64_t t0 = c * kQ;
        const uint16_t *zr = zg ? static_cast<const uint16_t *>(a.z) + ((ib * a.H + h) * kP + 32 * Pt + ln % 32) * a.L + t0
                                : nullptr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t4 = 32 * T + 8 * q + 4 * (ln / 32);
            if (VEC) zq[q] = zr && t4 + 4 <= a.L - t0 ? *reinterpret_cast<const uint2 *>(zr + t4) : make_uint2(0u, 0u);
            else zq[q] = zr ? raw4<uint16_t>(zr, t4, a.L - t0, false) : make_uint2(0u, 0u);
        }
    };
    // the chunk's scalars (every wavefront forms them from Δ; wavefront 0 publishes them) and its operands
    auto stage = [&]() {
        const float dt = widen(dtr);
        const float u = dt * (ah * kLog2e);
        const float abar = exp2_fast(u);
        const float beta = zoh_input_coef_log2(dt, u, abar, 1.0f / ah);
        const float cu = wave_prefix_sum(u);
        const float cend = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cu), 63));
        dec = exp2_fast(cend);
        if (w == 0) {
            s_cum[l] = cu;
            s_beta[l] = beta;
            s_w[l] = exp2_fast(cend - cu) * beta;
            s_et[l] = exp2_fast(cu);
        }
#pragma unroll
        for (int k = 0; k < CK; ++k) {
            *reinterpret_cast<uint4 *>(s_c + c_r(k) * NH + c_c(k)) = get4(cq, k);
            *reinterpret_cast<uint4 *>(s_b + l * NH + b_c(k)) = get4(bq, k);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) *reinterpret_cast<uint4 *>(s_x + x_r(k) * kMH + x_c(k)) = get4(xq, k);
    };
    // eight bf16 of an LDS row in accumulator row order: row[0 .. 3] and row[8 .. 11]
    auto pair8 = [](const uint16_t *row) {
        const uint2 u = *reinterpret_cast<const uint2 *>(row), v = *reinterpret_cast<const uint2 *>(row + 8);
        return make_uint4(u.x, u.y, v.x, v.y);
    };
    auto bf8 = [](const uint4 &v) { return __builtin_bit_cast(bf8v, v); };

    load_chunk(0);
    load_z(0);
    stage();
    load_chunk(a.nc > 1 ? 1 : 0);
    for (int64_t c = 0; c < a.nc; ++c) {
        const int64_t t0 = c * kQ;
        const int64_t lim = a.L - t0;
        lds_barrier();  // the chunk's operands and scalars; the previous chunk's product tiles are consumed

        // G = B Cᵀ for this wavefront's product tile (rows s = 32 gS .., columns t = 32 T ..)
        f16v g;  // formed by the wavefronts that own a product tile and read only by them
        if (gw) {
            g = f16v{};  // inside the branch: the other wavefront keeps no zeroed copy
            const uint16_t *arow = s_b + (32 * gS + lc) * NH + hi * HN, *brow = s_c + (32 * T + lc) * NH + hi * HN;
#pragma unroll
            for (int j = 0; j < HN / 8; ++j)
                g = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf8v *>(arow + 8 * j),
                                                            *reinterpret_cast<const bf8v *>(brow + 8 * j), g, 0, 0, 0);
        }
        // the entering state's part C_t·h_in over this wavefront's half of the states, for both step tiles
        // (C rows in accumulator order, Hᵀ as hi + lo); the partner's tile goes to it through LDS
        f16v y = {}, yo = {};
        {
            const uint16_t *crow = s_c + (32 * T + lc) * NH + n0 + 4 * hi;
            const uint16_t *corow = s_c + (32 * (1 - T) + lc) * NH + n0 + 4 * hi;
#pragma unroll
            for (int j = 0; j < NS; ++j)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    bf8v h8, l8;
                    split8(make_float4(acc[j][8 * kk], acc[j][8 * kk + 1], acc[j][8 * kk + 2], acc[j][8 * kk + 3]),
                           make_float4(acc[j][8 * kk + 4], acc[j][8 * kk + 5], acc[j][8 * kk + 6], acc[j][8 * kk + 7]),
                           h8, l8);
                    const bf8v co8 = bf8(pair8(corow + 32 * j + 16 * kk));
                    yo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(co8, h8, yo, 0, 0, 0);
                    yo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(co8, l8, yo, 0, 0, 0);
                    const bf8v c8 = bf8(pair8(crow + 32 * j + 16 * kk));
                    y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c8, h8, y, 0, 0, 0);
                    y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c8, l8, y, 0, 0, 0);
                }
            // e^{a c_t} on both partial sums here: the chunk's scalars are overwritten after the next barrier
            float4 *io = s_i + w * 4 * kWave + l;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 e4 = *reinterpret_cast<const float4 *>(s_et + 32 * T + 8 * q + 4 * hi);
                y[4 * q] *= e4.x; y[4 * q + 1] *= e4.y; y[4 * q + 2] *= e4.z; y[4 * q + 3] *= e4.w;
                const float4 eo = *reinterpret_cast<const float4 *>(s_et + 32 * (1 - T) + 8 * q + 4 * hi);
                io[q * kWave] = make_float4(yo[4 * q] * eo.x, yo[4 * q + 1] * eo.y, yo[4 * q + 2] * eo.z, yo[4 * q + 3] * eo.w);
            }
        }
        // the decayed product tile, split into bf16 hi and lo for the wavefronts that multiply it
        if (gw) {
            const float ct = s_cum[32 * T + lc];
            float m[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int s0 = 32 * gS + 8 * q + 4 * hi;
                const float4 cs = *reinterpret_cast<const float4 *>(s_cum + s0);
                const float4 bs = *reinterpret_cast<const float4 *>(s_beta + s0);
                const float csv[4] = {cs.x, cs.y, cs.z, cs.w}, bsv[4] = {bs.x, bs.y, bs.z, bs.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    m[4 * q + i] = s0 + i <= 32 * T + lc ? g[4 * q + i] * exp2_fast(ct - csv[i]) * bsv[i] : 0.0f;
            }
            uint4 *mo = s_m + (gS + T) * 4 * kWave + l;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf8v h8, l8;
                split8(make_float4(m[8 * kk], m[8 * kk + 1], m[8 * kk + 2], m[8 * kk + 3]),
                       make_float4(m[8 * kk + 4], m[8 * kk + 5], m[8 * kk + 6], m[8 * kk + 7]), h8, l8);
                mo[(2 * kk) * kWave] = __builtin_bit_cast(uint4, h8);
                mo[(2 * kk + 1) * kWave] = __builtin_bit_cast(uint4, l8);
            }
        }
        // x of channel p over the chunk in accumulator row order: xr[S][kk] holds steps 32 S + 16 kk + ..
        uint4 xr[2][2];
        {
            const uint16_t *xrow = s_x + p * kMH + 4 * hi;
#pragma unroll
            for (int S = 0; S < 2; ++S)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) xr[S][kk] = pair8(xrow + 32 * S + 16 * kk);
        }
        // the state update: Hᵀ ← e^{a c_end} Hᵀ + Bᵀ X_w, X_w[s][p] = x[p][s] e^{a(c_end − c_s)} β_s (hi + lo);
        // the Bᵀ operand (row n, k = s) is read down column n of B's rows
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][r] *= dec;
        {
            const uint16_t *bcol = s_b + (4 * hi) * NH + n0 + lc;
            auto col8 = [&](const uint16_t *c) {  // rows 0 .. 3 and 8 .. 11 of a column, packed in pairs
                uint32_t v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r0 = 2 * e + (e >= 2 ? 4 : 0);
                    v[e] = (uint32_t)c[r0 * NH] | ((uint32_t)c[(r0 + 1) * NH] << 16);
                }
                return make_uint4(v[0], v[1], v[2], v[3]);
            };
#pragma unroll
            for (int S = 0; S < 2; ++S)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int s0 = 32 * S + 16 * kk + 4 * hi;
                    const float4 w0 = *reinterpret_cast<const float4 *>(s_w + s0);
                    const float4 w1 = *reinterpret_cast<const float4 *>(s_w + s0 + 8);
                    const uint4 xv = xr[S][kk];
                    bf8v h8, l8;
                    split8(make_float4(bf16_lo(xv.x) * w0.x, bf16_hi(xv.x) * w0.y, bf16_lo(xv.y) * w0.z, bf16_hi(xv.y) * w0.w),
                           make_float4(bf16_lo(xv.z) * w1.x, bf16_hi(xv.z) * w1.y, bf16_lo(xv.w) * w1.z, bf16_hi(xv.w) * w1.w),
                           h8, l8);
#pragma unroll
                    for (int j = 0; j < NS; ++j) {
                        const bf8v b8 = bf8(col8(bcol + (32 * S + 16 * kk) * NH + 32 * j));
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b8, h8, acc[j], 0, 0, 0);
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b8, l8, acc[j], 0, 0, 0);
                    }
                }
        }
        lds_barrier();  // the product tiles and partial sums are written; every read of the operands is done

        // the next chunk's scalars and operands into LDS, then the loads of the one after. Done
        // unconditionally, with chunk indices clamped to the last chunk, so no branch joins the loads
        // in flight (a join made the compiler copy, and so wait for, the loaded registers); after the
        // last chunk these stage a chunk into LDS that nothing reads.
        stage();
        // the staging's LDS writes take the previous loads' registers before the next loads are issued
        // (otherwise both sets are live at once, and the prefetch arrays no longer fit in registers)
        asm volatile("" ::: "memory");
        load_chunk(c + 2 < a.nc ? c + 2 : a.nc - 1);
        // the partner's half of e^{a c_t} C_t·h_in
        {
            const float4 *ii = s_i + (w ^ 1) * 4 * kWave + l;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 o4 = ii[q * kWave];
                y[4 * q] += o4.x; y[4 * q + 1] += o4.y; y[4 * q + 2] += o4.z; y[4 * q + 3] += o4.w;
            }
        }
        // the chunk's own part: Σ_s M[t][s] x_s over the product tiles (S, T), S <= T (M as hi + lo)
#pragma unroll
        for (int S = 0; S < 2; ++S) {
            if (S > T) break;
            const uint4 *mi = s_m + (S + T) * 4 * kWave + l;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf8v x8 = bf8(xr[S][kk]);
                y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf8(mi[(2 * kk) * kWave]), x8, y, 0, 0, 0);
                y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf8(mi[(2 * kk + 1) * kWave]), x8, y, 0, 0, 0);
            }
        }
        // y = outputs + D x, times silu(z): channel p, steps 32 T + 8q + 4 hi .. +3 (registers 4q .. 4q+3)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int t4 = 32 * T + 8 * q + 4 * hi;
            if (t4 >= lim) continue;
            const uint4 xv = T == 0 ? xr[0][q / 2] : xr[1][q / 2];
            const uint32_t x0 = (q & 1) ? xv.z : xv.x, x1 = (q & 1) ? xv.w : xv.y;
            float v[4] = {y[4 * q] + dsk * bf16_lo(x0), y[4 * q + 1] + dsk * bf16_hi(x0),
                          y[4 * q + 2] + dsk * bf16_lo(x1), y[4 * q + 3] + dsk * bf16_hi(x1)};
            if (zg) {
                float zv[4];
                raw_elems(zq[q], zv);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] *= silu(zv[e]);
            }
            if (AM == 2) {
                uint2 pk;
                pk.x = (uint32_t)narrow<uint16_t>(v[0]) | ((uint32_t)narrow<uint16_t>(v[1]) << 16);
                pk.y = (uint32_t)narrow<uint16_t>(v[2]) | ((uint32_t)narrow<uint16_t>(v[3]) << 16);
                *reinterpret_cast<uint2 *>(yh + t0 + poff + 8 * q) = pk;
            } else if (VEC) {  // t4 < lim and lim a multiple of 8: the whole piece
                uint2 pk;
                pk.x = (uint32_t)narrow<uint16_t>(v[0]) | ((uint32_t)narrow<uint16_t>(v[1]) << 16);
                pk.y = (uint32_t)narrow<uint16_t>(v[2]) | ((uint32_t)narrow<uint16_t>(v[3]) << 16);
                *reinterpret_cast<uint2 *>(yg + t0 + t4) = pk;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (t4 + e < lim) yg[t0 + t4 + e] = narrow<uint16_t>(v[e]);
            }
        }
        load_z(c + 1 < a.nc ? c + 1 : a.nc - 1);
    }
    if (a.hT) {
        // the lane index behind an empty asm, so that these addresses are formed here and not kept
        // across the walk
        int ln = l;
        asm volatile("" : "+v"(ln));
        float *ht = a.hT + bh * (kP * N) + (int64_t)(32 * Pt + ln % 32) * N + n0;
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) ht[32 * j + d_row(r, ln)] = acc[j][r];
    }
}

template <typename T, int N>
hipError_t launch_walk(const SsdArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((ssd_scan_kernel<T, N>), dim3((unsigned)(a.b * a.H * (N / 64))), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fused(const SsdArgs &a, int64_t N, hipStream_t stream) {
    const dim3 grid((unsigned)(a.b * a.H));
    const bool vec = a.vec && a.vec8 && a.vec_bc16;
    const bool whole = vec && a.L % kQ == 0 && kP * a.L < (INT64_C(1) << 31);
    if (N == 64 && whole) hipLaunchKernelGGL((ssd_fused_kernel<64, 2>), grid, dim3(kThreads), 0, stream, a);
    else if (N == 64 && vec) hipLaunchKernelGGL((ssd_fused_kernel<64, 1>), grid, dim3(kThreads), 0, stream, a);
    else if (N == 64) hipLaunchKernelGGL((ssd_fused_kernel<64, 0>), grid, dim3(kThreads), 0, stream, a);
    else if (N == 128 && whole) hipLaunchKernelGGL((ssd_fused_kernel<128, 2>), grid, dim3(kThreads), 0, stream, a);
    else if (N == 128 && vec) hipLaunchKernelGGL((ssd_fused_kernel<128, 1>), grid, dim3(kThreads), 0, stream, a);
    else if (N == 128) hipLaunchKernelGGL((ssd_fused_kernel<128, 0>), grid, dim3(kThreads), 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_state_walk(const SsdArgs &a, int64_t N, bool bf16, hipStream_t stream) {
    if (N == 64) return bf16 ? launch_walk<uint16_t, 64>(a, stream) : launch_walk<float, 64>(a, stream);
    if (N == 128) return bf16 ? launch_walk<uint16_t, 128>(a, stream) : launch_walk<float, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace ssd
}  // namespace ssm
