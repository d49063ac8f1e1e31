// scan_fwd.hip — prefill selective scan for gfx950: fused ZOH discretisation + recurrence + readout
// + gate/skip epilogue, an aggregate pass and a chunk-carry pass for sequences split in time.
//
// Method (page "Mambaとは？Transformer以外の系列モデル", sections 状態空間モデルを一つの式から理解する
// and Mambaの核心は入力依存のDelta、B、C; page "State Space Models（SSM）とMamba" §2.2, §4.2–§4.3):
//   Ā = exp(Δ·A), B̄ = (Ā − 1)/A · B, h_t = Ā h_{t−1} + B̄ x_t, y_t = C_t·h_t + D x_t, y ← y·silu(z).
//
// Mapping onto CDNA4:
//   * One lane owns one channel (b, d) and walks time in order, so the recurrence never leaves
//     registers and needs no cross-lane traffic. A workgroup holds 64 channels of one batch row
//     and 1, 2 or 4 wavefronts; each wavefront owns a contiguous group of `NPL` states of every
//     channel, so B_t and C_t for that group are wave-uniform and come in through scalar loads.
//   * x and Δ rows are read as coalesced 16-byte chunks (time is contiguous in memory), widened to
//     fp32 once and staged in LDS, double-buffered; each lane then reads its own row.
//   * Per (t, n) the fast path issues one exp and six fp32 VALU operations. With the scaled state
//     s = A·h the ZOH input needs no division:  s_t = s_{t−1} + (Ā − 1)·(s_{t−1} + B x),
//     and the readout is Σ_n (C_n / A_n)·s_n. Ā − 1 is exact in fp32 (Sterbenz) and damps the
//     rounding of s + Bx. States of channels with |A| < 2^-10 use an unscaled path whose input
//     coefficient comes from the series of (e^v − 1)/v near v = 0 (the A = 0 limit is Δ·B).
//   * The readout partials of the wavefronts meet in LDS; the epilogue (sum, + D·x, · silu(z),
//     rounding) runs time-major so that y rows are written coalesced.
//   * Long sequences are cut into time segments (page "Mambaとは？…", section Selective Scanは
//     選択機構そのものではない: affine maps (A, b) compose associatively). An aggregate pass gives
//     each segment's (Π Ā, end state from zero); a carry pass chains them per (b, d, n); the output
//     pass then rescans every segment from its true carry-in.
#include "device_common.h"
#include "launch.h"

namespace ssm {
namespace {

constexpr int kPitch = kTile + 4;             // floats per LDS row: 16-byte pad, conflict-free b128
constexpr int kRowsF = kGroupRows * kPitch;   // floats per [64][pitch] LDS plane
constexpr float kSafeAbsA = 1.0f / 1024.0f;   // |A| below this takes the unscaled path

struct FwdArgs {
    const void *x, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z;
    void *y;
    float *final_state;
    const float *init_state;  // segment 0 carry-in (nullable)
    const float *h_in;        // carry-in of segments 1.. : [n_seg-1][b][d][N] (output pass)
    float *agg_P;             // aggregate pass outputs [n_seg-1][b][d][N]
    float *agg_E;
    int64_t b, d, L, N;
    int64_t seg_len;
    int64_t n_db;             // channel blocks per batch row
    int vec_rows;             // x/Δ/z rows allow 16-byte loads at every tile
    int vec_bc;               // B/C tile runs allow 16-byte loads
};

template <typename T> struct Chunk;                 // 16 bytes of one row
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
__device__ __forceinline__ void put_chunk_regs(float *dst, const uint4 &v);
template <>
__device__ __forceinline__ void put_chunk_regs<float>(float *dst, const uint4 &v) {
    dst[0] = __uint_as_float(v.x); dst[1] = __uint_as_float(v.y);
    dst[2] = __uint_as_float(v.z); dst[3] = __uint_as_float(v.w);
}
template <>
__device__ __forceinline__ void put_chunk_regs<uint16_t>(float *dst, const uint4 &v) {
    dst[0] = bf16_lo(v.x); dst[1] = bf16_hi(v.x); dst[2] = bf16_lo(v.y); dst[3] = bf16_hi(v.y);
    dst[4] = bf16_lo(v.z); dst[5] = bf16_hi(v.z); dst[6] = bf16_lo(v.w); dst[7] = bf16_hi(v.w);
}

// Load one chunk (E consecutive elements of a row or run) with bounds; elements at or past
// `t_end` are 0.
template <typename T>
__device__ __forceinline__ uint4 get_chunk(const T *__restrict__ row, int64_t t, int64_t t_end,
                                           bool row_ok, bool vec) {
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

// LDS helpers -------------------------------------------------------------------------------

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

template <int U>
__device__ __forceinline__ void lds_put(float *p, const float (&v)[U]) {
    if constexpr (U == 4) *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    else if constexpr (U == 2) *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
    else *p = v[0];
}

// Scan one LDS tile for this wavefront's NPL states.
//   xrow, drow : this lane's x and Δ for the tile (LDS, fp32)
//   Bn, Cn     : the tile's B and C planes [kTile][NPAD] (LDS, fp32), offset to state n0; the
//                reads are wave-uniform, so every lane receives the same values
//   prow       : this lane's readout partials for the tile (LDS), output pass only
//   dskip      : D·x is added to this wave's partial (nonzero on wave 0 only)
// SAFE selects the unscaled path; AGG drops the readout (aggregate pass).
//
// The tile is walked in sub-tiles of U = 8 / NPL timesteps (1 for NPL >= 8). Each step issues the LDS reads of the
// NEXT sub-tile before computing the current one. LDS operations complete in order, so the wait
// for the current sub-tile leaves the prefetch in flight.
template <int NPL, int NPAD, bool SAFE, bool AGG>
__device__ __forceinline__ void scan_tile(const float *xrow, const float *drow, const float *Bn,
                                          const float *Cn, float *prow, float dskip,
                                          const float (&a2)[NPL], const float (&Av)[NPL],
                                          const float (&ia)[NPL], float (&s)[NPL], float &dsum) {
    constexpr int U = NPL >= 8 ? 1 : 8 / NPL;
    constexpr int NSUB = kTile / U;  // even
    struct Sub {
        float x[U], d[U], B[U][NPL], C[U][NPL];
    };
    auto load_sub = [&](int u, Sub &o) {
        lds_get<U>(xrow + u * U, o.x);
        lds_get<U>(drow + u * U, o.d);
#pragma unroll
        for (int k = 0; k < U; ++k) {
#pragma unroll
            for (int j = 0; j < NPL; j += 4) {
                const float4 b = *reinterpret_cast<const float4 *>(Bn + (u * U + k) * NPAD + j);
                o.B[k][j] = b.x; o.B[k][j + 1] = b.y; o.B[k][j + 2] = b.z; o.B[k][j + 3] = b.w;
                if constexpr (!AGG) {
                    const float4 c = *reinterpret_cast<const float4 *>(Cn + (u * U + k) * NPAD + j);
                    o.C[k][j] = c.x; o.C[k][j + 1] = c.y; o.C[k][j + 2] = c.z; o.C[k][j + 3] = c.w;
                }
            }
        }
    };
    auto compute_sub = [&](int u, const Sub &c) {
        float yv[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const float xt = c.x[k], dt = c.d[k];
            float acc = dskip * xt;
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
                const float abar = exp2_fast(dt * a2[j]);
                if constexpr (!SAFE) {
                    const float pre = __builtin_fmaf(c.B[k][j], xt, s[j]);  // s + B x
                    s[j] = __builtin_fmaf(abar - 1.0f, pre, s[j]);          // s + (Ā − 1)(s + B x)
                    if constexpr (!AGG) acc = __builtin_fmaf(c.C[k][j] * ia[j], s[j], acc);
                } else {
                    const float kc = zoh_input_coef(dt, Av[j], abar, ia[j]);
                    s[j] = __builtin_fmaf(abar, s[j], kc * (c.B[k][j] * xt));  // Ā h + B̄ x
                    if constexpr (!AGG) acc = __builtin_fmaf(c.C[k][j], s[j], acc);
                }
            }
            if constexpr (AGG) dsum += dt;
            yv[k] = acc;
        }
        if constexpr (!AGG) lds_put<U>(prow + u * U, yv);
    };
    Sub s0, s1;
    load_sub(0, s0);
#pragma unroll 1
    for (int u = 0; u < NSUB; u += 2) {
        load_sub(u + 1, s1);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the arithmetic
        compute_sub(u, s0);
        load_sub(u + 2 < NSUB ? u + 2 : u + 1, s0);  // the last pass re-reads a sub-tile it has
        __builtin_amdgcn_sched_barrier(0);
        compute_sub(u + 1, s1);
    }
}

// The kernel --------------------------------------------------------------------------------
//
// One workgroup: 64 channels (one per lane) of batch row bi, time segment `seg`, GW wavefronts
// (wave w owns states [w*NPL, (w+1)*NPL)). Per tile of kTile timesteps:
//   scan (LDS only) -> barrier -> store the prefetched next tile into LDS, epilogue of this tile,
//   issue the global loads of the tile after next -> barrier.
// The tile's x and Δ rows, and its B and C rows (one contiguous run of kTile*N elements each),
// are fetched one tile ahead into registers with 16-byte loads and widened to fp32 on the way
// into LDS, so the scan never touches global memory.
template <typename T, int NPL, int GW, bool AGG>
__global__ __launch_bounds__(kWave *GW) void scan_fwd_kernel(FwdArgs a) {
    constexpr int E = Chunk<T>::kElems;
    constexpr int kThreads = kWave * GW;
    constexpr int kChunksPerRow = kTile / E;
    constexpr int kCPT = kGroupRows * kChunksPerRow / kThreads;                 // x/Δ chunks per thread
    constexpr int kEPT = kGroupRows * kTile / kThreads;                         // epilogue elements per thread
    constexpr int NPAD = NPL * GW;                                              // states held in LDS per timestep
    constexpr int kBCF = kTile * NPAD;                                          // floats per B or C plane
    constexpr int kBCT = (kBCF / E + kThreads - 1) / kThreads;                  // B/C chunks per thread
    __shared__ __attribute__((aligned(16))) float xs[kRowsF];
    __shared__ __attribute__((aligned(16))) float dsh[kRowsF];
    __shared__ __attribute__((aligned(16))) float Bs[kBCF];
    __shared__ __attribute__((aligned(16))) float Cs[AGG ? 4 : kBCF];
    __shared__ __attribute__((aligned(16))) float part[AGG ? 4 : GW * kRowsF];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int64_t ncb = a.b * a.n_db;
    const int64_t blk = blockIdx.x;
    const int64_t seg = blk / ncb;
    const int64_t cb = blk - seg * ncb;
    const int64_t bi = cb / a.n_db;
    const int64_t d0 = (cb - bi * a.n_db) * kGroupRows;
    const int64_t t_begin = seg * a.seg_len;
    const int64_t t_end = (t_begin + a.seg_len < a.L) ? t_begin + a.seg_len : a.L;
    const int ntiles = (int)((t_end - t_begin + kTile - 1) / kTile);
    const int64_t bd = a.b * a.d;
    const int N = (int)a.N;

    const T *__restrict__ xg = static_cast<const T *>(a.x);
    const T *__restrict__ dg = static_cast<const T *>(a.delta);
    const T *__restrict__ zg = static_cast<const T *>(a.z);
    const T *__restrict__ Bg = static_cast<const T *>(a.B) + bi * a.L * a.N;
    const T *__restrict__ Cg = static_cast<const T *>(a.C) + bi * a.L * a.N;
    T *__restrict__ yg = static_cast<T *>(a.y);

    // ---- per-lane channel constants for this wave's state group ----
    const int64_t ch = d0 + lane;
    const bool ch_ok = ch < a.d;
    const int n0 = wave * NPL;
    const int nvalid = (N - n0) < NPL ? (N - n0) : NPL;  // <= 0 for a wave past the last state
    const int64_t row = bi * a.d + ch;
    float Av[NPL], a2[NPL], ia[NPL], s[NPL];
    bool small_a = false;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const bool ok = ch_ok && j < nvalid;
        const float av = ok ? a.A[ch * a.N + n0 + j] : -1.0f;  // idle states: A = −1 with B = C = 0
        Av[j] = av;
        a2[j] = av * kLog2e;
        ia[j] = 1.0f / av;
        small_a |= __builtin_fabsf(av) < kSafeAbsA;
        float h0 = 0.0f;  // the aggregate pass always scans its segment from the zero state
        if constexpr (!AGG) {
            if (ok) {
                if (seg == 0) {
                    if (a.init_state) h0 = a.init_state[row * a.N + n0 + j];
                } else {
                    h0 = a.h_in[((seg - 1) * bd + row) * a.N + n0 + j];
                }
            }
        }
        s[j] = h0;
    }
    const bool safe = __any(small_a);  // wave-uniform choice of path
    if (!safe) {
#pragma unroll
        for (int j = 0; j < NPL; ++j) s[j] *= Av[j];  // scaled state s = A·h
    }
    const float dskip = (!AGG && wave == 0 && ch_ok && a.D) ? a.D[ch] : 0.0f;

    // ---- tile prefetch (registers) and its store into LDS ----
    uint4 px[kCPT], pd[kCPT], pb[kBCT], pc[kBCT];
    auto load_tile = [&](int64_t t0) {
#pragma unroll
        for (int i = 0; i < kCPT; ++i) {
            const int c = tid + i * kThreads;
            const int r = c / kChunksPerRow;
            const int64_t tt = t0 + (c % kChunksPerRow) * E;
            const bool rok = d0 + r < a.d;
            const int64_t off = rok ? (bi * a.d + d0 + r) * a.L : 0;
            px[i] = get_chunk<T>(xg + off, tt, t_end, rok, a.vec_rows);
            pd[i] = get_chunk<T>(dg + off, tt, t_end, rok, a.vec_rows);
        }
        // B and C rows t0 .. t0 + kTile − 1 form one run of kTile * N elements; rows at or past L
        // are not read (their Δ is 0, so their values do not matter: zeros keep them finite).
        const int64_t rows = (a.L - t0) < kTile ? (a.L - t0) : kTile;
        const int64_t nel = rows * a.N;
#pragma unroll
        for (int i = 0; i < kBCT; ++i) {
            const int c = tid + i * kThreads;
            const int64_t e0 = (int64_t)c * E;
            pb[i] = get_chunk<T>(Bg + t0 * a.N, e0, nel, e0 < (int64_t)kBCF, a.vec_bc);
            if constexpr (!AGG) pc[i] = get_chunk<T>(Cg + t0 * a.N, e0, nel, e0 < (int64_t)kBCF, a.vec_bc);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < kCPT; ++i) {
            const int c = tid + i * kThreads;
            const int r = c / kChunksPerRow;
            const int col = (c % kChunksPerRow) * E;
            put_chunk<T>(xs + r * kPitch + col, px[i]);
            put_chunk<T>(dsh + r * kPitch + col, pd[i]);
        }
#pragma unroll
        for (int i = 0; i < kBCT; ++i) {
            const int c = tid + i * kThreads;
            const int e0 = c * E;
            if (e0 >= kTile * N) continue;
            if (N == NPAD) {  // the run maps onto the [kTile][NPAD] plane one to one
                put_chunk<T>(Bs + e0, pb[i]);
                if constexpr (!AGG) put_chunk<T>(Cs + e0, pc[i]);
            } else {          // scatter element by element; columns N .. NPAD−1 stay zero
                float vb[E], vc[E];
                put_chunk_regs<T>(vb, pb[i]);
                if constexpr (!AGG) put_chunk_regs<T>(vc, pc[i]);
#pragma unroll
                for (int q = 0; q < E; ++q) {
                    const int e = e0 + q;
                    if (e < kTile * N) {
                        const int t = e / N, n = e - t * N;
                        Bs[t * NPAD + n] = vb[q];
                        if constexpr (!AGG) Cs[t * NPAD + n] = vc[q];
                    }
                }
            }
        }
    };

    if (N != NPAD) {  // padding columns of the B/C planes must read as zero
        for (int i = tid; i < kBCF; i += kThreads) {
            Bs[i] = 0.0f;
            if constexpr (!AGG) Cs[i] = 0.0f;
        }
        __syncthreads();
    }

    float zv[kEPT];
    auto load_z = [&](int64_t t0) {
        if constexpr (!AGG) {
#pragma unroll
            for (int i = 0; i < kEPT; ++i) {
                const int e = tid + i * kThreads;
                const int r = e / kTile;
                const int64_t tg = t0 + (e % kTile);
                zv[i] = 0.0f;
                if (zg && d0 + r < a.d && tg < t_end) zv[i] = widen(zg[(bi * a.d + d0 + r) * a.L + tg]);
            }
        }
    };

    float dsum = 0.0f;
    load_tile(t_begin);
    store_tile();
    if (ntiles > 1) load_tile(t_begin + kTile);
    load_z(t_begin);
    __syncthreads();

    const float *xrow = xs + lane * kPitch;
    const float *drow = dsh + lane * kPitch;
    float *prow = AGG ? part : part + wave * kRowsF + lane * kPitch;
#pragma unroll 1
    for (int it = 0; it < ntiles; ++it) {
        const int64_t t0 = t_begin + (int64_t)it * kTile;
        if (!safe)
            scan_tile<NPL, NPAD, false, AGG>(xrow, drow, Bs + n0, Cs + n0, prow, dskip, a2, Av, ia, s, dsum);
        else
            scan_tile<NPL, NPAD, true, AGG>(xrow, drow, Bs + n0, Cs + n0, prow, dskip, a2, Av, ia, s, dsum);
        __syncthreads();

        if (it + 1 < ntiles) store_tile();
        if constexpr (!AGG) {
            // Epilogue, time-major: consecutive lanes take consecutive timesteps of one row.
#pragma unroll
            for (int i = 0; i < kEPT; ++i) {
                const int e = tid + i * kThreads;
                const int r = e / kTile;
                const int col = e % kTile;
                const int64_t tg = t0 + col;
                if (d0 + r < a.d && tg < t_end) {
                    float v = part[r * kPitch + col];
#pragma unroll
                    for (int w = 1; w < GW; ++w) v += part[w * kRowsF + r * kPitch + col];
                    if (zg) v *= silu(zv[i]);
                    yg[(bi * a.d + d0 + r) * a.L + tg] = narrow<T>(v);
                }
            }
        }
        if (it + 2 < ntiles) load_tile(t0 + 2 * kTile);
        if (it + 1 < ntiles) load_z(t0 + kTile);
        __syncthreads();
    }

    // ---- segment results ----
    if (ch_ok) {
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            if (j >= nvalid) continue;
            const float h = safe ? s[j] : s[j] * ia[j];
            const int64_t idx = row * a.N + n0 + j;
            if constexpr (AGG) {
                a.agg_P[seg * bd * a.N + idx] = exp2_fast(a2[j] * dsum);  // Π Ā = exp(A ΣΔ)
                a.agg_E[seg * bd * a.N + idx] = h;                        // end state from zero
            } else {
                if (a.final_state && t_end == a.L) a.final_state[idx] = h;
            }
        }
    }
}

// Chunk carry: h_in[k] = P[k−1]·h_in[k−1] + E[k−1] per (b, d, n), h_in[0] = initial state.
__global__ __launch_bounds__(256) void carry_kernel(const float *__restrict__ P, const float *__restrict__ Eend,
                                                    float *__restrict__ Hin, const float *__restrict__ init,
                                                    int64_t bdn, int n_seg) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= bdn) return;
    float h = init ? init[i] : 0.0f;
    for (int k = 0; k + 1 < n_seg; ++k) {
        h = __builtin_fmaf(P[k * bdn + i], h, Eend[k * bdn + i]);
        Hin[k * bdn + i] = h;
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

template <typename T, int NPL, int GW>
hipError_t launch_typed(const FwdArgs &args, int n_seg, int64_t ncb, const FwdLaunch &p, hipStream_t stream) {
    if (n_seg > 1) {
        const int64_t grid = (int64_t)(n_seg - 1) * ncb;
        hipLaunchKernelGGL((scan_fwd_kernel<T, NPL, GW, true>), dim3((unsigned)grid), dim3(kWave * GW), 0, stream, args);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t bdn = p.b * p.d * p.N;
        hipLaunchKernelGGL(carry_kernel, dim3((unsigned)((bdn + 255) / 256)), dim3(256), 0, stream, args.agg_P,
                           args.agg_E, const_cast<float *>(args.h_in), p.init_state, bdn, n_seg);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.ev_begin) {
        hipError_t e = hipEventRecord(p.ev_begin, stream);
        if (e != hipSuccess) return e;
    }
    const int64_t grid = (int64_t)n_seg * ncb;
    hipLaunchKernelGGL((scan_fwd_kernel<T, NPL, GW, false>), dim3((unsigned)grid), dim3(kWave * GW), 0, stream, args);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.ev_end) e = hipEventRecord(p.ev_end, stream);
    return e;
}

template <typename T>
hipError_t dispatch_shape(const FwdArgs &args, int n_seg, int64_t ncb, const FwdLaunch &p, hipStream_t stream) {
#define SSM_CASE(NPL_, GW_) \
    if (p.states_per_wave == NPL_ && p.waves == GW_) return launch_typed<T, NPL_, GW_>(args, n_seg, ncb, p, stream);
    SSM_CASE(4, 1) SSM_CASE(4, 2) SSM_CASE(4, 4)
    SSM_CASE(8, 1) SSM_CASE(8, 2) SSM_CASE(8, 4)
    SSM_CASE(16, 1) SSM_CASE(16, 2) SSM_CASE(16, 4)
#undef SSM_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan_fwd(const FwdLaunch &p, hipStream_t stream) {
    FwdArgs a{};
    a.x = p.x; a.delta = p.delta; a.A = p.A; a.B = p.B; a.C = p.C; a.D = p.D; a.z = p.z; a.y = p.y;
    a.final_state = p.final_state;
    a.init_state = p.init_state;
    a.b = p.b; a.d = p.d; a.L = p.L; a.N = p.N;
    a.seg_len = p.seg_len;
    a.n_db = (p.d + kGroupRows - 1) / kGroupRows;
    const int64_t esize = p.bf16 ? 2 : 4;
    auto aligned16 = [](const void *q) { return q == nullptr || (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
    a.vec_rows = ((p.L * esize) % 16 == 0) && aligned16(p.x) && aligned16(p.delta) && aligned16(p.z);
    // a tile's B/C run starts at element (bi*L + t0)*N with t0 a multiple of 32
    a.vec_bc = ((p.L * p.N * esize) % 16 == 0) && aligned16(p.B) && aligned16(p.C);
    if (p.n_seg > 1) {
        const int64_t per = (int64_t)(p.n_seg - 1) * p.b * p.d * p.N;
        a.agg_P = p.scratch;
        a.agg_E = p.scratch + per;
        a.h_in = p.scratch + 2 * per;
    }
    const int64_t ncb = p.b * a.n_db;
    if (p.bf16) return dispatch_shape<uint16_t>(a, p.n_seg, ncb, p, stream);
    return dispatch_shape<float>(a, p.n_seg, ncb, p, stream);
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace ssm
