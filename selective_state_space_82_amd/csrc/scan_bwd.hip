// scan_bwd.hip — gradients of the prefill selective scan for gfx950.
//
// The forward map (page "Mambaとは？Transformer以外の系列モデル", section 状態空間モデルを一つの式から
// 理解する; page "State Space Models（SSM）とMamba" §2.2, §4.2) is, per (b, d, n),
//   h_t = Ā_t h_{t−1} + β_t B_t x_t,  Ā = e^{Δa},  β = (e^{Δa} − 1)/a,
//   ys_t = Σ_n C_tn h_tn + D x_t,  y_t = ys_t·silu(z_t).
// Its gradients follow by the chain rule in reverse time, with the adjoint λ_t = ∂L/∂h_t:
//   λ_t = dys_t C_t + κ_{t+1},  κ_t = Ā_t λ_t  (κ after the last step: the final-state gradient),
//   dĀ_t = λ_t h_{t−1},  dβ_t = λ_t B_t x_t,  ∂Ā/∂Δ = aĀ, ∂Ā/∂a = ΔĀ, ∂β/∂Δ = Ā,
//   ∂β/∂a = (ΔĀ − β)/a (Δ²/2 at a = 0).
// The forward states are not stored: the same page's hardware-aware section recomputes them in the
// backward pass. Here a forward pass leaves the state entering every K-th step (K = 32 / NPL, at
// least 4, so the K·NPL states of a chunk fit a lane's registers with two wavefronts per SIMD); the
// gradient pass restarts from each checkpoint, recomputes K steps forward, then walks them backward.
//
// Mapping onto CDNA4 (as in the prefill kernel): one wavefront per unit = 64/G channels of one
// batch row over one time segment, G lanes per channel with NPL states each.
//   * Time segments run in parallel: the adjoint recurrence κ_t = Ā_t(dys_t C_t + κ_{t+1}) is
//     affine, so a reverse aggregate pass gives each segment (Π Ā, κ at its start from κ = 0 at its
//     end) and each gradient wavefront chains the aggregates of the segments after its own.
//   * Per-step sums over a channel's states (the readout ys, dx, dΔ) are DPP butterflies over the G
//     lanes. dB and dC sum over channels: the wave's partials go through LDS, are summed over its
//     channels there, and are added to the outputs with float atomics (so their low bits depend on
//     the order in which waves finish). dA and dD are per-lane sums added atomically at the end.
//   * Tiles of 16 steps of x, Δ, z and dy rows (and the B, C runs) are prefetched one tile ahead
//     (in reverse time order) into registers and staged in the wave's LDS, z and dy as the gate's two
//     factors (computed once per element); dx, dΔ, dz collect in LDS and leave a row segment at a time.
#include "device_common.h"
#include "launch.h"
#include "tile_common.h"

namespace ssm {
namespace {

constexpr int kBT = 16;  // steps per tile in the gradient passes

struct BwdArgs {
    const void *x, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z, *dy;
    const float *dh_final;
    const float *ckpt;      // [b][d][n_ck][N]: state entering step k * ck_len
    const float *rP, *rE;   // reverse aggregates of segments 1 .. S−1, [S−1][b][d][N]
    float *rP_out, *rE_out;
    void *dx, *ddelta, *dz;
    float *dA, *dB, *dC, *dD, *dh0;
    int64_t b, d, L, N;
    int64_t seg_len, n_cw, n_ck;
    int n_seg, ck_len;
    int vec_rows, vec_bc, vec_state;
};

// ∂β/∂a = (Δ Ā − β)/a, from its series Δ²(1/2 + v/3 + v²/8 + v³/30) when |v| = |Δa| < 1/16.
__device__ __forceinline__ float dbeta_da(float dt, float u, float abar, float beta, float inv_a) {
    const float v = u * 0.69314718055994530942f;
    const float series = dt * dt * __builtin_fmaf(v, __builtin_fmaf(v, __builtin_fmaf(v, 1.0f / 30.0f, 0.125f), 1.0f / 3.0f), 0.5f);
    const float direct = (dt * abar - beta) * inv_a;
    return __builtin_fabsf(v) < 0.0625f ? series : direct;
}

// REV: reverse aggregate pass (no gradients; segments 1 .. S−1), else the gradient pass. β always takes
// the series of (e^v − 1)/v where |v| = |ΔA| < 1/16: (Ā − 1)/A from a float Ā near 1 would carry a
// relative error of about 2^-24/|ΔA| there, which slow channels (small |ΔA| for many steps) expose.
template <typename T, int G, int NPL, bool REV>
__global__ __launch_bounds__(kWave, 2) void scan_bwd_kernel(BwdArgs a) {
    constexpr int E = Chunk<T>::kElems;
    constexpr int kPitch = kBT + 4;
    constexpr int CW = kWave / G;
    constexpr int NPAD = G * NPL;
    constexpr int K = (32 / NPL) < 4 ? 4 : 32 / NPL;    // steps per checkpoint chunk
    // with 4 states per lane, Ā and β of the chunk's last KH steps stay in registers from the forward
    // recomputation to the walk back, which computes them again for the other steps (register budget)
    constexpr bool kKeep = NPL <= 4;
    constexpr int KH = K / 2;
    constexpr int kRowChunks = kBT / E;                  // 16-byte chunks per row per tile
    constexpr int kXC = (CW * kRowChunks + kWave - 1) / kWave;
    constexpr int kBF = kBT * NPAD;
    constexpr int kBC = (kBF / E + kWave - 1) / kWave;
    constexpr int kRG = 4;                               // steps per dB/dC reduction group
    constexpr int kRed = kRG * 2 * NPAD;                 // dB, dC outputs per group (over channels)
    constexpr int kRedPerLane = (kRed + kWave - 1) / kWave;
    static_assert(kBT % K == 0 && K % kRG == 0, "chunks tile the tile, reduction groups tile the chunk");
    __shared__ __attribute__((aligned(16))) float xs[CW * kPitch];
    __shared__ __attribute__((aligned(16))) float ds[CW * kPitch];
    __shared__ __attribute__((aligned(16))) float zs[REV ? 4 : CW * kPitch];  // the gate's dz factor
    __shared__ __attribute__((aligned(16))) float gs[CW * kPitch];   // ∂L/∂ys (dy through the gate)
    __shared__ __attribute__((aligned(16))) float Bs[REV ? 4 : kBF];
    __shared__ __attribute__((aligned(16))) float Cs[kBF];
    __shared__ __attribute__((aligned(16))) float outs[REV ? 4 : 3 * CW * kPitch];  // dx, dΔ, dz
    __shared__ __attribute__((aligned(16))) float red[REV ? 4 : kRG * 2 * CW * NPAD];

    const int lane = threadIdx.x;
    const int c = lane / G;
    const int g = lane % G;
    const uint32_t ncb = (uint32_t)(a.b * a.n_cw);
    const uint32_t ublk = (uint32_t)blockIdx.x + (REV ? ncb : 0u);  // REV covers segments 1 .. S−1
    const int64_t seg = ublk / ncb;
    const uint32_t cb = ublk - (uint32_t)seg * ncb;
    const int64_t bi = cb / (uint32_t)a.n_cw;
    const int64_t d0 = (int64_t)(cb - (uint32_t)bi * (uint32_t)a.n_cw) * CW;
    const int64_t t_begin = seg * a.seg_len;
    const int64_t t_end = (t_begin + a.seg_len < a.L) ? t_begin + a.seg_len : a.L;
    const int ntiles = (int)((t_end - t_begin + kBT - 1) / kBT);
    const int64_t bd = a.b * a.d;
    const int N = (int)a.N;

    const T *__restrict__ xg = static_cast<const T *>(a.x);
    const T *__restrict__ dg = static_cast<const T *>(a.delta);
    const T *__restrict__ zg = static_cast<const T *>(a.z);
    const T *__restrict__ gg = static_cast<const T *>(a.dy);
    const T *__restrict__ Bg = static_cast<const T *>(a.B) + bi * a.L * a.N;
    const T *__restrict__ Cg = static_cast<const T *>(a.C) + bi * a.L * a.N;
    const bool gate = zg != nullptr;

    const int64_t ch = d0 + c;
    const bool ch_ok = ch < a.d;
    const int n0 = g * NPL;
    const int nvalid = (N - n0) < NPL ? (N - n0) : NPL;
    const int64_t row = bi * a.d + ch;
    const int64_t sidx = row * a.N + n0;
    float Av[NPL], a2[NPL], ia[NPL], gA[NPL];
    // The adjoint carried to the previous step, in fp64: it sums dys·C over the whole remaining sequence,
    // undamped where Δ·A is small, and an fp32 carry would round at 2^-24 of its size on every step; the
    // part that survives in dΔ = Σ_n λ_n B_n x (+ …) shows where that sum over states cancels. For the
    // same reason the decay is applied as κ = λ + (Ā − 1)·λ with Ā − 1 accurate in relative terms (the
    // series near ΔA = 0): a float Ā itself is only within 2^-25 of its value, and that error compounds
    // over the sequence. fp64 adds and multiplies issue at the fp32 rate on this GPU.
    double kap[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const bool ok = ch_ok && j < nvalid;
        const float av = load_or(a.A, ch * a.N + n0 + j, ok, -1.0f);
        Av[j] = av;
        a2[j] = av * kLog2e;
        ia[j] = 1.0f / av;
        gA[j] = 0.0f;
        kap[j] = 0.0;
    }
    auto load_state = [&](const float *base, float (&o)[NPL]) {
        if (a.vec_state) {
#pragma unroll
            for (int j = 0; j < NPL; j += 4) {
                const bool ok = ch_ok && j + 4 <= nvalid;
                const float4 v = *reinterpret_cast<const float4 *>(base + (ok ? sidx + j : 0));
                o[j] = ok ? v.x : 0.0f; o[j + 1] = ok ? v.y : 0.0f; o[j + 2] = ok ? v.z : 0.0f; o[j + 3] = ok ? v.w : 0.0f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NPL; ++j) o[j] = load_or(base, sidx + j, ch_ok && j < nvalid, 0.0f);
        }
    };
    if constexpr (!REV) {
        // adjoint entering this segment from the right: the final-state gradient, carried through
        // the aggregates of every later segment (κ ← P_j κ + E_j for j = S−1 down to seg+1)
        if (a.dh_final) {
            float k0[NPL];
            load_state(a.dh_final, k0);
#pragma unroll
            for (int q = 0; q < NPL; ++q) kap[q] = k0[q];
        }
        for (int64_t j = a.n_seg - 1; j > seg; --j) {
            float P[NPL], Ej[NPL];
            load_state(a.rP + (j - 1) * bd * a.N, P);
            load_state(a.rE + (j - 1) * bd * a.N, Ej);
#pragma unroll
            for (int q = 0; q < NPL; ++q) kap[q] = __builtin_fma((double)P[q], kap[q], (double)Ej[q]);
        }
    }
    const float dskip = (!REV && a.D) ? load_or(a.D, ch, ch_ok, 0.0f) : 0.0f;
    float gD = 0.0f;

    // ---- tile staging (reverse order: tile it + 1 is processed before tile it) ----
    uint4 px[kXC], pd[kXC], pz[kXC], pg[kXC], pb[kBC], pc[kBC];
    auto load_tile = [&](int64_t t0) {
        int ln = lane;
        asm volatile("" : "+v"(ln));  // form the addresses here rather than keep them across the walk
#pragma unroll
        for (int i = 0; i < kXC; ++i) {
            const int k = ln + i * kWave;
            const int r = k / kRowChunks;
            const int64_t tt = t0 + (k % kRowChunks) * E;
            const bool rok = k < CW * kRowChunks && d0 + r < a.d;
            const int64_t off = rok ? (bi * a.d + d0 + r) * a.L : 0;
            if constexpr (!REV) px[i] = get_chunk<T>(xg + off, tt, t_end, rok, a.vec_rows);
            pd[i] = get_chunk<T>(dg + off, tt, t_end, rok, a.vec_rows);
            if (gate) pz[i] = get_chunk<T>(zg + off, tt, t_end, rok, a.vec_rows);
            pg[i] = get_chunk<T>(gg + off, tt, t_end, rok, a.vec_rows);
        }
        const int64_t rows = (a.L - t0) < kBT ? (a.L - t0) : kBT;
        const int64_t nel = rows * a.N;
#pragma unroll
        for (int i = 0; i < kBC; ++i) {
            const int64_t e0 = (int64_t)(ln + i * kWave) * E;
            const bool ok = e0 < (int64_t)kBT * N;
            if constexpr (!REV) pb[i] = get_chunk<T>(Bg + t0 * a.N, e0, nel, ok, a.vec_bc);
            pc[i] = get_chunk<T>(Cg + t0 * a.N, e0, nel, ok, a.vec_bc);
        }
    };
    auto store_tile = [&]() {
        int ln = lane;
        asm volatile("" : "+v"(ln));  // as in load_tile
#pragma unroll
        for (int i = 0; i < kXC; ++i) {
            const int k = ln + i * kWave;
            if (k >= CW * kRowChunks) break;
            const int r = k / kRowChunks;
            const int col = (k % kRowChunks) * E;
            if constexpr (!REV) put_chunk<T>(xs + r * kPitch + col, px[i]);
            put_chunk<T>(ds + r * kPitch + col, pd[i]);
            if (gate) {
                // the gate's factors, once per element rather than on each of a channel's G lanes:
                // gs <- dy·silu(z) = ∂L/∂ys, zs <- dy·σ(z)·(1 + z(1 − σ(z))), which times ys is ∂L/∂z
                float zv[E], gv[E], fz[E];
                chunk_to_regs<T>(zv, pz[i]);
                chunk_to_regs<T>(gv, pg[i]);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float sg = __builtin_amdgcn_rcpf(1.0f + exp2_fast(-kLog2e * zv[e]));
                    fz[e] = gv[e] * sg * __builtin_fmaf(zv[e], 1.0f - sg, 1.0f);
                    gv[e] = gv[e] * zv[e] * sg;
                }
#pragma unroll
                for (int e = 0; e < E; e += 4) {
                    *reinterpret_cast<float4 *>(gs + r * kPitch + col + e) = make_float4(gv[e], gv[e + 1], gv[e + 2], gv[e + 3]);
                    if constexpr (!REV)
                        *reinterpret_cast<float4 *>(zs + r * kPitch + col + e) = make_float4(fz[e], fz[e + 1], fz[e + 2], fz[e + 3]);
                }
            } else {
                put_chunk<T>(gs + r * kPitch + col, pg[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < kBC; ++i) {
            const int e0 = (ln + i * kWave) * E;
            if (e0 >= kBT * N) break;
            if (N == NPAD) {
                if constexpr (!REV) put_chunk<T>(Bs + e0, pb[i]);
                put_chunk<T>(Cs + e0, pc[i]);
            } else {
                float vb[E], vc[E];
                if constexpr (!REV) chunk_to_regs<T>(vb, pb[i]);
                chunk_to_regs<T>(vc, pc[i]);
#pragma unroll
                for (int q = 0; q < E; ++q) {
                    const int e = e0 + q;
                    if (e < kBT * N) {
                        const int t = e / N, n = e - t * N;
                        if constexpr (!REV) Bs[t * NPAD + n] = vb[q];
                        Cs[t * NPAD + n] = vc[q];
                    }
                }
            }
        }
    };
    if (N != NPAD) {
        for (int i = lane; i < kBF; i += kWave) {
            if constexpr (!REV) Bs[i] = 0.0f;
            Cs[i] = 0.0f;
        }
    }

    const float *xrow = xs + c * kPitch;
    const float *drow = ds + c * kPitch;
    const float *zrow = zs + c * kPitch;
    const float *grow = gs + c * kPitch;
    const float *Bn = Bs + n0;
    const float *Cn = Cs + n0;
    auto dys_of = [&](int t) { return grow[t]; };  // ∂L/∂ys_t: dy_t·silu(z_t) with a gate, else dy_t

    // ---- reverse aggregate pass: κ from zero at the segment's end back to its start ----
    if constexpr (REV) {
        float dsum = 0.0f;
        load_tile(t_begin + (int64_t)(ntiles - 1) * kBT);
        store_tile();
        if (ntiles > 1) load_tile(t_begin + (int64_t)(ntiles - 2) * kBT);
        wave_sync();
#pragma unroll 1
        for (int it = ntiles - 1; it >= 0; --it) {
#pragma unroll 4
            for (int t = kBT - 1; t >= 0; --t) {
                const float dt = drow[t];
                const float dys = dys_of(t);
                float Cv[NPL];
#pragma unroll
                for (int j = 0; j < NPL; j += 4) {
                    const float4 cv = *reinterpret_cast<const float4 *>(Cn + t * NPAD + j);
                    Cv[j] = cv.x; Cv[j + 1] = cv.y; Cv[j + 2] = cv.z; Cv[j + 3] = cv.w;
                }
#pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    const float u = dt * a2[j];
                    const double lam = kap[j] + (double)(dys * Cv[j]);
                    kap[j] = __builtin_fma((double)expm1_log2(u, exp2_fast(u)), lam, lam);
                }
                dsum += dt;
            }
            if (it > 0) {
                wave_sync();
                store_tile();
                wave_sync();
            }
            if (it > 1) load_tile(t_begin + (int64_t)(it - 2) * kBT);
        }
        if (ch_ok) {
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
                if (j >= nvalid) continue;
                const int64_t o = (seg - 1) * bd * a.N + sidx + j;
                a.rP_out[o] = exp2_fast(a2[j] * dsum);
                a.rE_out[o] = (float)kap[j];
            }
        }
        return;
    }

    // ---- gradient pass ----
    T *const dxg = static_cast<T *>(a.dx);
    T *const ddg = static_cast<T *>(a.ddelta);
    T *const dzg = static_cast<T *>(a.dz);
    float *const outx = outs;
    float *const outd = outs + CW * kPitch;
    float *const outz = outs + 2 * CW * kPitch;
    // this lane's dB/dC partials for step k of a reduction group: red[((k*2 + q)*CW + c)*NPAD + n]
    auto red_at = [&](int k, int q) { return red + ((k * 2 + q) * CW + c) * NPAD + n0; };
    // sum the group's partials over the wave's channels and add them to dB/dC (steps t0g .. t0g+3)
    auto reduce_group = [&](int64_t t0g) {
        wave_sync();
#pragma unroll
        for (int i = 0; i < kRedPerLane; ++i) {
            const int o = lane + i * kWave;  // o = (k*2 + q)*NPAD + n
            if (o >= kRed) break;
            const int n = o % NPAD;
            const int kq = o / NPAD;
            const int k = kq / 2, q = kq % 2;
            float sum = 0.0f;
#pragma unroll
            for (int cc = 0; cc < CW; ++cc) sum += red[(kq * CW + cc) * NPAD + n];
            const int64_t t = t0g + k;
            if (n < N && t < t_end) {
                float *dst = (q == 0 ? a.dB : a.dC) + (bi * a.L + t) * a.N + n;
                unsafeAtomicAdd(dst, sum);
            }
        }
        wave_sync();
    };
    // flush the dx, dΔ, dz rows of tile t0 (16 steps, valid < t_end): lane l stores steps
    // 4(l % 4) .. +3 of row l / 4 of each of the three outputs
    static_assert(CW * 4 <= kWave * 4, "rows per flush");
    const int fr = lane / 4, fq = (lane % 4) * 4;
    const bool f_ok = fr < CW && d0 + fr < a.d;
    const int64_t f_off = f_ok ? (bi * a.d + d0 + fr) * a.L : 0;
    auto flush_out = [&](int64_t t0) {
        if (!f_ok) return;
#pragma unroll
        for (int which = 0; which < 3; ++which) {
            if (which == 2 && !gate) break;
            T *dst = (which == 0 ? dxg : which == 1 ? ddg : dzg) + f_off + t0 + fq;
            const float *src = outs + which * CW * kPitch + fr * kPitch + fq;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (t0 + fq + e < t_end) dst[e] = narrow<T>(src[e]);
        }
    };

    const int64_t t_last = t_begin + (int64_t)(ntiles - 1) * kBT;
    load_tile(t_last);
    store_tile();
    if (ntiles > 1) load_tile(t_last - kBT);
    wave_sync();
    // the state entering chunk kc: ckpt[row][kc][n0 ..], zeros for idle lanes
    auto load_ckpt = [&](int64_t kc, float (&o)[NPL]) {
        const int64_t idx = (row * a.n_ck + kc) * a.N + n0;
        if (a.vec_state) {
#pragma unroll
            for (int j = 0; j < NPL; j += 4) {
                const bool ok = ch_ok && j + 4 <= nvalid;
                const float4 v = *reinterpret_cast<const float4 *>(a.ckpt + (ok ? idx + j : 0));
                o[j] = ok ? v.x : 0.0f; o[j + 1] = ok ? v.y : 0.0f; o[j + 2] = ok ? v.z : 0.0f; o[j + 3] = ok ? v.w : 0.0f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NPL; ++j) o[j] = load_or(a.ckpt, idx + j, ch_ok && j < nvalid, 0.0f);
        }
    };
    // The chunks are walked in descending order, kc_last down to kc_first; the checkpoint of the next
    // one is loaded a chunk ahead (raw, from an always-valid address, and masked only when used), so
    // its latency hides behind a chunk of arithmetic.
    const int64_t kc_first = t_begin / K, kc_last = (t_end - 1) / K;
    bool ck_ok[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) ck_ok[j] = ch_ok && (a.vec_state ? (j / 4) * 4 + 4 <= nvalid : j < nvalid);
    float hn[NPL];
    auto load_ckpt_raw = [&](int64_t kc) {
        const int64_t idx = (row * a.n_ck + kc) * a.N + n0;
        if (a.vec_state) {
#pragma unroll
            for (int j = 0; j < NPL; j += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(a.ckpt + (ck_ok[j] ? idx + j : 0));
                hn[j] = v.x; hn[j + 1] = v.y; hn[j + 2] = v.z; hn[j + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NPL; ++j) hn[j] = a.ckpt[ck_ok[j] ? idx + j : 0];
        }
    };
    load_ckpt_raw(kc_last);
#pragma unroll 1
    for (int it = ntiles - 1; it >= 0; --it) {
        const int64_t t0 = t_begin + (int64_t)it * kBT;
#pragma unroll 1
        for (int m = kBT / K - 1; m >= 0; --m) {
            const int tc = m * K;  // chunk start within the tile
            if (t0 + tc >= t_end) continue;  // all padding (no checkpoint there; nothing would change)
            // state entering the chunk (written by the forward pass)
            const int64_t kc = (t0 + tc) / K;
            float h[NPL];
#pragma unroll
            for (int j = 0; j < NPL; ++j) h[j] = ck_ok[j] ? hn[j] : 0.0f;
            if (kc > kc_first) load_ckpt_raw(kc - 1);
            // forward recomputation of the chunk: hs[k] = state after step tc + k
            float hs[K][NPL];
            float ab_k[kKeep ? KH : 1][kKeep ? NPL : 1], be_k[kKeep ? KH : 1][kKeep ? NPL : 1];
            // Both walks read a step's operands from LDS one step ahead of their use, so the wait for
            // them falls behind a step of arithmetic instead of stalling at the start of each step.
            float fx = xrow[tc], fd = drow[tc];
            float4 fb[NPL / 4];
#pragma unroll
            for (int j = 0; j < NPL; j += 4) fb[j / 4] = *reinterpret_cast<const float4 *>(Bn + tc * NPAD + j);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int t = tc + k;
                const float xt = fx, dt = fd;
                float4 bcur[NPL / 4];
#pragma unroll
                for (int j = 0; j < NPL; j += 4) bcur[j / 4] = fb[j / 4];
                if (k + 1 < K) {
                    fx = xrow[t + 1];
                    fd = drow[t + 1];
#pragma unroll
                    for (int j = 0; j < NPL; j += 4) fb[j / 4] = *reinterpret_cast<const float4 *>(Bn + (t + 1) * NPAD + j);
                }
#pragma unroll
                for (int j = 0; j < NPL; j += 4) {
                    const float4 bv = bcur[j / 4];
                    const float bq[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float u = dt * a2[j + q];
                        const float abar = exp2_fast(u);
                        const float beta = zoh_input_coef_log2(dt, u, abar, ia[j + q]);
                        const float hp = k == 0 ? h[j + q] : hs[k - 1][j + q];
                        hs[k][j + q] = __builtin_fmaf(abar, hp, beta * (bq[q] * xt));
                        if constexpr (kKeep) {
                            if (k >= K - KH) {
                                ab_k[k - (K - KH)][j + q] = abar;
                                be_k[k - (K - KH)][j + q] = beta;
                            }
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);  // one step at a time: keeps the live ranges short
            }
            // backward over the chunk. The fence makes the walk re-read its operands from LDS
            // rather than keep the forward walk's copies alive in registers.
            wave_sync();
            float wx, wd, wg, wz;
            float4 wb[NPL / 4], wc[NPL / 4];
            auto read_step = [&](int t) {
                wx = xrow[t];
                wd = drow[t];
                wg = grow[t];
                wz = gate ? zrow[t] : 0.0f;
#pragma unroll
                for (int j = 0; j < NPL; j += 4) {
                    wb[j / 4] = *reinterpret_cast<const float4 *>(Bn + t * NPAD + j);
                    wc[j / 4] = *reinterpret_cast<const float4 *>(Cn + t * NPAD + j);
                }
            };
            read_step(tc + K - 1);
#pragma unroll
            for (int k = K - 1; k >= 0; --k) {
                const int t = tc + k;
                const float xt = wx;
                float dt = wd;
                const float dyt = wg, zt = wz;
                float Bv[NPL], Cv[NPL];
#pragma unroll
                for (int j = 0; j < NPL; j += 4) {
                    const float4 bv = wb[j / 4], cv = wc[j / 4];
                    Bv[j] = bv.x; Bv[j + 1] = bv.y; Bv[j + 2] = bv.z; Bv[j + 3] = bv.w;
                    Cv[j] = cv.x; Cv[j + 1] = cv.y; Cv[j + 2] = cv.z; Cv[j + 3] = cv.w;
                }
                if (k > 0) read_step(t - 1);
                // where not kept, Ā and β are recomputed here rather than kept from the forward walk
                // (K·NPL pairs of registers); the empty asm hides that they are the same values
                if (!kKeep || k < K - KH) asm volatile("" : "+v"(dt));
                // readout ys_t (for dz) and the gated output gradient
                float ysp = 0.0f;
#pragma unroll
                for (int j = 0; j < NPL; ++j) ysp = __builtin_fmaf(Cv[j], hs[k][j], ysp);
                const float ys = __builtin_fmaf(dskip, xt, group_sum<G>(ysp));
                const float dys = dyt;      // the staged ∂L/∂ys
                const float dzt = ys * zt;  // zero without a gate (zt reads as 0 then)
                float gx = 0.0f, gd = 0.0f;
                const int kr = k % kRG;
                float *rb = red_at(kr, 0);
                float *rc = red_at(kr, 1);
#pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    const float u = dt * a2[j];
                    float abar, beta;
                    if (kKeep && k >= K - KH) {
                        abar = ab_k[kKeep ? k - (K - KH) : 0][j];
                        beta = be_k[kKeep ? k - (K - KH) : 0][j];
                    } else {
                        abar = exp2_fast(u);
                        beta = zoh_input_coef_log2(dt, u, abar, ia[j]);
                    }
                    const float hp = k == 0 ? h[j] : hs[k - 1][j];
                    const double lam64 = kap[j] + (double)(dys * Cv[j]);
                    const float lam = (float)lam64;
                    const float dab = lam * hp;                 // ∂L/∂Ā_t
                    const float dbe = lam * (Bv[j] * xt);       // ∂L/∂β_t
                    rb[j] = lam * beta * xt;                    // dB partial (this channel)
                    rc[j] = dys * hs[k][j];                     // dC partial
                    gx = __builtin_fmaf(lam * beta, Bv[j], gx);
                    gd = __builtin_fmaf(__builtin_fmaf(dab, Av[j], dbe), abar, gd);
                    gA[j] = __builtin_fmaf(dab * abar, dt, __builtin_fmaf(dbe, dbeta_da(dt, u, abar, beta, ia[j]), gA[j]));
                    kap[j] = __builtin_fma((double)(beta * Av[j]), lam64, lam64);  // λ + (Ā − 1)·λ
                }
                gx = __builtin_fmaf(dys, dskip, group_sum<G>(gx));
                gd = group_sum<G>(gd);
                gD = __builtin_fmaf(dys, xt, gD);
                // the G lanes of a channel hold the same sums and store them to the same place (no
                // branch: a divergent one per step would split the unrolled walk into small blocks)
                outx[c * kPitch + t] = gx;
                outd[c * kPitch + t] = gd;
                outz[c * kPitch + t] = dzt;
                if (kr == 0) reduce_group(t0 + t);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wave_sync();
        flush_out(t0);
        if (it > 0) {
            wave_sync();
            store_tile();
            wave_sync();
        }
        if (it > 1) load_tile(t0 - 2 * kBT);
    }

    // ---- per-lane sums: dA over (b, t), dD over (b, t), the initial-state gradient ----
    if (ch_ok) {
#pragma unroll
        for (int j = 0; j < NPL; ++j)
            if (j < nvalid) unsafeAtomicAdd(a.dA + ch * a.N + n0 + j, gA[j]);
        if (g == 0 && a.dD) unsafeAtomicAdd(a.dD + ch, gD);
        if (seg == 0 && a.dh0) {
#pragma unroll
            for (int j = 0; j < NPL; ++j)
                if (j < nvalid) a.dh0[sidx + j] = (float)kap[j];
        }
    }
}

// Clears up to four buffers (the summed gradients) in one launch: element i of the concatenation.
struct ZeroList {
    float *p[4];
    int64_t n[4];
};

__global__ __launch_bounds__(256) void zero_kernel(ZeroList z, int64_t total) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t k = i;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (k < z.n[b]) {
                z.p[b][k] = 0.0f;
                break;
            }
            k -= z.n[b];
        }
    }
}

hipError_t zero4(ZeroList z, hipStream_t stream) {
    int64_t total = 0;
    for (int b = 0; b < 4; ++b) {
        if (!z.p[b] || z.n[b] < 0) z.n[b] = 0;
        total += z.n[b];
    }
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream, z, total);
    return hipGetLastError();
}

template <typename T, int G, int NPL>
hipError_t launch_bwd_typed(BwdArgs args, int64_t ncb, int n_seg, hipStream_t stream) {
    if (n_seg > 1) {
        hipLaunchKernelGGL((scan_bwd_kernel<T, G, NPL, true>), dim3((unsigned)((n_seg - 1) * ncb)), dim3(kWave), 0,
                           stream, args);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((scan_bwd_kernel<T, G, NPL, false>), dim3((unsigned)(n_seg * ncb)), dim3(kWave), 0, stream,
                       args);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_bwd(const BwdArgs &args, int G, int NPL, int64_t ncb, int n_seg, hipStream_t stream) {
#define SSM_BCASE(G_, NPL_) \
    if (G == G_ && NPL == NPL_) return launch_bwd_typed<T, G_, NPL_>(args, ncb, n_seg, stream);
    SSM_BCASE(4, 4) SSM_BCASE(4, 8) SSM_BCASE(4, 16)
#undef SSM_BCASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan_bwd(const BwdLaunch &p, hipStream_t stream) {
    const int npl = p.states_per_lane;
    const int ck = ckpt_len(npl);
    const int64_t n_ck = (p.L + ck - 1) / ck;
    const int64_t fwd_scratch = scratch_floats(p.n_seg, p.b, p.d, p.N);
    float *ckpt = p.scratch + fwd_scratch;
    float *rP = ckpt + p.b * p.d * n_ck * p.N;
    float *rE = rP + (int64_t)(p.grad_n_seg - 1) * p.b * p.d * p.N;

    const ZeroList zl{{p.dA, p.dB, p.dC, p.dD}, {p.d * p.N, p.b * p.L * p.N, p.b * p.L * p.N, p.dD ? p.d : 0}};
    hipError_t e = zero4(zl, stream);
    if (e != hipSuccess) return e;

    // forward pass that leaves the checkpoints (no outputs)
    FwdLaunch f{};
    f.x = p.x; f.delta = p.delta; f.A = p.A; f.B = p.B; f.C = p.C; f.D = p.D; f.z = p.z;
    f.y = nullptr; f.final_state = nullptr; f.init_state = p.init_state;
    f.b = p.b; f.d = p.d; f.L = p.L; f.N = p.N; f.bf16 = p.bf16;
    f.lanes_per_channel = p.lanes_per_channel; f.states_per_lane = npl;
    f.seg_len = p.seg_len; f.n_seg = p.n_seg; f.scratch = p.scratch;
    f.ckpt = ckpt; f.ck_len = ck;
    e = launch_scan_fwd(f, stream);
    if (e != hipSuccess) return e;

    BwdArgs a{};
    a.x = p.x; a.delta = p.delta; a.A = p.A; a.B = p.B; a.C = p.C; a.D = p.D; a.z = p.z; a.dy = p.dy;
    a.dh_final = p.d_final_state; a.ckpt = ckpt; a.rP = rP; a.rE = rE; a.rP_out = rP; a.rE_out = rE;
    a.dx = p.dx; a.ddelta = p.ddelta; a.dz = p.dz; a.dA = p.dA; a.dB = p.dB; a.dC = p.dC; a.dD = p.dD;
    a.dh0 = p.d_init_state;
    a.b = p.b; a.d = p.d; a.L = p.L; a.N = p.N; a.seg_len = p.grad_seg_len; a.n_seg = p.grad_n_seg;
    const int cw = kWave / p.lanes_per_channel;
    a.n_cw = (p.d + cw - 1) / cw;
    a.n_ck = n_ck; a.ck_len = ck;
    const int64_t esize = p.bf16 ? 2 : 4;
    auto al16 = [](const void *q) { return q == nullptr || (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
    a.vec_rows = ((p.L * esize) % 16 == 0) && al16(p.x) && al16(p.delta) && al16(p.z) && al16(p.dy);
    a.vec_bc = ((p.L * p.N * esize) % 16 == 0) && al16(p.B) && al16(p.C);
    a.vec_state = (p.N % 4 == 0) && al16(p.d_final_state) && al16(p.scratch) && al16(ckpt) && al16(rP) && al16(rE);
    const int64_t ncb = p.b * a.n_cw;
    if (p.bf16) return dispatch_bwd<uint16_t>(a, p.lanes_per_channel, npl, ncb, p.grad_n_seg, stream);
    return dispatch_bwd<float>(a, p.lanes_per_channel, npl, ncb, p.grad_n_seg, stream);
}

}  // namespace ssm
