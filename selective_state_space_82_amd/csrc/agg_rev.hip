// agg_rev.hip — the aggregate pass of a time-split prefill for gfx950: each segment's end state from zero
// and its decay product, by a backward walk that stops once the decay back to the step it has reached is
// negligible.
//
// Method (page "Mambaとは？Transformer以外の系列モデル", section Selective Scanは選択機構そのものではない: the
// per-step maps h ↦ Ā h + B̄ x compose associatively; page "State Space Models（SSM）とMamba" §2.2 for the
// ZOH terms). A segment composes to h ↦ P·h + E with
//   P = Π_t Ā_t = exp(A·ΣΔ),   E = Σ_t R_t·B̄_t x_t,   R_t = Π_{u>t} Ā_u,
// E being the segment's end state from the zero state. Walking the segment backward, R_t is at hand at
// every step (R ← R·Ā_t after using it), so E accumulates R_t·B̄_t x_t. In the scaled form s = A·h used by
// the output pass, A·B̄ = Ā − 1, so the walk adds R·(Ā − 1)·B x and scales by 1/A once at the end.
//
// Truncation. Once R ≤ 2^-24 for every state a wavefront holds, the steps not yet walked contribute exactly
// R·h_t, where h_t is the state at the step reached (from zero at the segment start): at most 2^-24·|h_t|,
// fp32's unit roundoff times |h_t|. Holding h_t in fp32 at that step already errs by that much, and that
// error reaches the segment end decayed by the same R, so dropping the rest costs no more than one
// rounding of the state the output pass itself carries. The walk stops there (a state with A ≥ 0 never
// decays and is walked to the segment start). The decay rate |A_n|·Δ differs by an order of magnitude across n (A_n ≈ −(n + 1)
// under Mamba's initialisation), so a wavefront holds one group of four states of 64 channels (a lane per
// channel, its four states in registers): the groups of fast states stop after a few dozen steps.
//
// Work unit = (segment, batch row, block of 64 channels, state group). The groups of a (segment, row,
// block) read the same x and Δ rows over nested ranges, so they are numbered to land on one XCD
// (workgroups go to the 8 XCDs in turn), where the longest walk's reads serve the others from that XCD's
// L2; and group-major, so the long walks start first. A tile of x and Δ (64 rows × 64 bytes) is loaded
// with 16-byte loads, four lanes per row, and staged through LDS in the storage type; each lane then reads
// its own row, and the group's B_t from a broadcast plane. The walk is software-pipelined: the exponentials
// of step t − 1 are formed in the same stretch of code as the accumulation of step t, which carries only R
// and E from step to step, so a wavefront has eight independent chains in flight.
//
// P = exp(A·ΣΔ): each wavefront writes it for its own states, exact when its walk reached the segment start,
// and 0 when the walk stopped early (every state it holds had decayed below 2^-24 by then, and P is no larger
// than that decay times the carried-in state's own decay over the steps not walked; the term P·h_in is then
// within one fp32 rounding of a state there, as the truncated part of E is). So no step beyond a walk's
// stop is read.
//
// Split walk. When the caller gives E2 (a carry pass follows), group 0's walk, the longest, is split
// between two wavefronts per unit by the same composition: the later part walks the segment's last tiles
// into E; the earlier part sums Δ over those tiles, starts with R = exp(A·ΣΔ) (the decay from the segment
// end back to there) and walks on below them into E2, and forms P. E + E2 is the whole walk's sum.
//
// Per (t, n) the common path issues one exp and five fp32 operations: u, R·Ā (which is also R's update),
// B·x, the difference R·Ā − R = R·(Ā − 1), and the accumulation. Tiles are classified per wavefront as in
// the output pass: where some channel's Δ-sum over the tile is small against 1/|A|, Ā − 1 comes from the
// cubic series of 2^u − 1 near 0, and a wavefront holding a state at the A = 0 limit (|A| < 2^-64) takes
// B̄ = Δ·B with R = 1 there.
//
// The prefill launcher takes this pass for segments of 1024 steps or more; below that a segment rarely
// outlasts the slow states' decay, and the forward aggregate pass, whose wavefronts are equally long,
// finishes sooner than the walks of the slowest group running alone on their SIMDs.
#include "device_common.h"
#include "launch.h"
#include "tile_common.h"

namespace ssm {
namespace {

constexpr float kStopRel = 5.960464478e-8f;    // 2^-24
constexpr float kZeroAbs = 5.421010862e-20f;   // 2^-64: |A| below this takes the A = 0 limit
// 2^u − 1 = u·(c1 + u·(c2 + u·c3)) + O(u^4) with c_k = ln(2)^k / k!: relative error below 4e-6 for |u| < 1/16
constexpr float kPow2C1 = 0.693147180559945f;
constexpr float kPow2C2 = 0.240226506959101f;
constexpr float kPow2C3 = 0.0555041086648216f;
constexpr int kXcds = 8;                       // XCDs that take workgroups in turn
constexpr int kRowWords = 16;                  // 64 bytes of a row per tile
constexpr int kPitch = kRowWords + 1;          // words per LDS row (odd: lanes reading one word each never share a bank)

// Steps per tile: 64 bytes of a row.
template <typename T> constexpr int agg_tile() { return sizeof(T) == 2 ? 32 : 16; }
// Mean |Δ·A·log2 e| per step below which a tile takes Ā − 1 from its series (as the output pass does).
template <typename T> constexpr float agg_class_mean_u() { return sizeof(T) == 2 ? 1.0f / 4096.0f : 1.0f / 128.0f; }

struct AggArgs {
    const void *x, *delta;
    const float *A;
    const void *B;
    float *P, *E;          // [n_seg − 1][b][d][N]
    float *E2;             // the split walk's earlier sums (states 0..3), or null: no split
    int split_tiles;       // tiles at the segment end walked by the later part of group 0 (split walk)
    int64_t b, d, L, N;
    int64_t seg_len;
    int64_t n_cb;          // blocks of 64 channels per batch row
    int64_t n_units;       // (n_seg − 1)·b·n_cb
    int n_grp;             // groups of four states: ceil(N / 4)
    int vec_rows, vec_bc;
};

// Step k of a tile from this lane's LDS row (a word holds one fp32 or two bf16 steps).
template <typename T> __device__ __forceinline__ float row_step(const uint32_t *row, int k);
template <> __device__ __forceinline__ float row_step<float>(const uint32_t *row, int k) {
    return __uint_as_float(row[k]);
}
template <> __device__ __forceinline__ float row_step<uint16_t>(const uint32_t *row, int k) {
    const uint32_t w = row[k >> 1];
    return (k & 1) ? bf16_hi(w) : bf16_lo(w);
}

// NP: floats per row of the B plane (16 for N <= 16, else 64).
template <typename T, int NP>
__global__ __launch_bounds__(kWave, 3) void agg_rev_kernel(AggArgs a) {
    constexpr int kNP = NP;
    constexpr int kT = agg_tile<T>();
    constexpr int E = Chunk<T>::kElems;
    constexpr int kBCh = (kT * kNP / E + kWave - 1) / kWave;  // 16-byte chunks of the B run per lane (at most)
    __shared__ uint32_t xs[kWave * kPitch];
    __shared__ uint32_t ds[kWave * kPitch];
    __shared__ __attribute__((aligned(16))) float Bs[kT * kNP];

    const int lane = threadIdx.x;
    const int N = (int)a.N;
    // workgroup -> (state group, unit), group-major: the long walks of group 0 are dispatched first and the
    // short ones fill in around them; with the unit count padded to a multiple of 8, the groups of unit u
    // all land on u's XCD
    const uint32_t blk = blockIdx.x;
    const uint32_t nu8 = (uint32_t)((a.n_units + kXcds - 1) / kXcds * kXcds);
    const int slot = (int)(blk / nu8);
    const int64_t u = blk - (uint32_t)slot * nu8;
    if (u >= a.n_units) return;  // padding of the unit count (wave-uniform)
    // With the split walk, slot 0 is group 0's earlier part and slot 1 its later part (the longest walks
    // first); the other groups follow. part: 0 whole walk, 1 earlier part, 2 later part.
    const bool split = a.E2 != nullptr;
    const int grp = split ? (slot < 2 ? 0 : slot - 1) : slot;
    const int part = split && slot < 2 ? (slot == 0 ? 1 : 2) : 0;
    const uint32_t ncb = (uint32_t)(a.b * a.n_cb);
    const int64_t seg = u / ncb;
    const uint32_t cb = (uint32_t)(u - seg * ncb);
    const int64_t bi = cb / (uint32_t)a.n_cb;
    const int64_t c0 = (int64_t)(cb - (uint32_t)bi * (uint32_t)a.n_cb) * kWave;
    const int64_t ch = c0 + lane;
    const bool ch_ok = ch < a.d;
    const int n0 = grp * 4;
    const int64_t t_begin = seg * a.seg_len;
    const int64_t t_end = (t_begin + a.seg_len < a.L) ? t_begin + a.seg_len : a.L;
    const int ntiles = (int)((t_end - t_begin + kT - 1) / kT);

    const T *__restrict__ xg = static_cast<const T *>(a.x);
    const T *__restrict__ dg = static_cast<const T *>(a.delta);
    const T *__restrict__ Bg = static_cast<const T *>(a.B) + bi * a.L * a.N;

    // this lane's four states: log2-scaled A, the result's scale (1/A, or 1 at the A = 0 limit)
    float a2[4], isc[4], R[4], Eacc[4];
    bool live[4], zero[4];
    bool zero_any = false;
    float amin = __builtin_inff();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        live[j] = ch_ok && n0 + j < N;
        const float av = load_or(a.A, ch * a.N + n0 + j, live[j], -1.0f);
        zero[j] = __builtin_fabsf(av) < kZeroAbs;
        a2[j] = zero[j] ? 0.0f : av * kLog2e;
        isc[j] = zero[j] ? 1.0f : 1.0f / av;
        R[j] = 1.0f;
        Eacc[j] = 0.0f;
        zero_any |= live[j] && zero[j];
        if (live[j]) amin = __builtin_fminf(amin, __builtin_fabsf(a2[j]));
    }
    const bool wave_zero = __any(zero_any);
    // a tile whose Δ-sum falls below thr_sum runs accurate (+inf at A = 0: always; 0 for an idle lane: never)
    const float thr_sum = (float)kT * agg_class_mean_u<T>() / amin;

    // ---- staging: chunk q = lane % 4 of rows lane / 4 + 16 i (i < 4) of x and Δ; the tile's B run ----
    const int sr = lane / 4, sq = lane % 4;
    uint4 px[4], pd[4], pb[kBCh];
    auto load_tile = [&](int64_t t0, bool with_xb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = c0 + sr + 16 * i;
            const bool ok = r < a.d;
            const int64_t off = ok ? (bi * a.d + r) * a.L : 0;
            if (with_xb) px[i] = get_chunk<T>(xg + off, t0 + sq * E, t_end, ok, a.vec_rows);
            pd[i] = get_chunk<T>(dg + off, t0 + sq * E, t_end, ok, a.vec_rows);
        }
        if (with_xb) {
            const int64_t rows = (a.L - t0) < kT ? (a.L - t0) : kT;
            const int64_t nel = rows * a.N;
#pragma unroll
            for (int i = 0; i < kBCh; ++i) {
                const int64_t e0 = (int64_t)(lane + i * kWave) * E;
                pb[i] = get_chunk<T>(Bg + t0 * a.N, e0, nel, e0 < (int64_t)kT * N, a.vec_bc);
            }
        }
    };
    auto store_tile = [&](bool with_xb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int w = (sr + 16 * i) * kPitch + sq * 4;
            if (with_xb) {
                xs[w] = px[i].x; xs[w + 1] = px[i].y; xs[w + 2] = px[i].z; xs[w + 3] = px[i].w;
            }
            ds[w] = pd[i].x; ds[w + 1] = pd[i].y; ds[w + 2] = pd[i].z; ds[w + 3] = pd[i].w;
        }
        if (with_xb) {
            int l = lane;
            asm volatile("" : "+v"(l));  // form the addresses here rather than keep them across the walk
#pragma unroll
            for (int i = 0; i < kBCh; ++i) {  // the run into the [kT][kNP] plane (columns N .. stay zero)
                const int e0 = (l + i * kWave) * E;
                if (e0 >= kT * N) break;
                if (N % E == 0) {  // the chunk lies within one row
                    const int t = e0 / N, n = e0 - t * N;
                    put_chunk<T>(Bs + t * kNP + n, pb[i]);
                } else {
                    float v[E];
                    chunk_to_regs<T>(v, pb[i]);
#pragma unroll
                    for (int q = 0; q < E; ++q) {
                        const int e = e0 + q;
                        if (e < kT * N) Bs[(e / N) * kNP + e % N] = v[q];
                    }
                }
            }
        }
    };
    const uint32_t *xrow = xs + lane * kPitch;
    const uint32_t *drow = ds + lane * kPitch;
    const float *Bq = Bs + n0;
    // Δ-sum of this lane's row over the staged tile (the padding past the segment reads as 0)
    auto row_dsum = [&]() {
        float sum = 0.0f;
#pragma unroll
        for (int k = 0; k < kT; ++k) sum += row_step<T>(drow, k);
        return sum;
    };

    // One tile, backward, software-pipelined: the coefficients of step k − 1 are formed while step k
    // accumulates. Mode 0: Ā − 1 as computed; 1: from its series near 0; 2: 1 and the A = 0 limit (B̄ = Δ·B
    // there, with no decay).
    auto walk_tile = [&](auto mode_c) {
        constexpr int MODE = decltype(mode_c)::value;
        float cin[4], cdec[4];  // input and decay coefficients (Ā − 1) of the step being accumulated
        auto coefs = [&](int k, float (&ci)[4], float (&cd)[4]) {
            const float dt = row_step<T>(drow, k);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float uu = dt * a2[j];
                if constexpr (MODE == 0) {  // Ā alone (the accumulation forms R·Ā − R)
                    ci[j] = cd[j] = exp2_fast(uu);
                    continue;
                }
                float em1 = exp2_fast(uu) - 1.0f;
                if constexpr (MODE >= 1) {
                    const float p = __builtin_fmaf(__builtin_fmaf(uu, kPow2C3, kPow2C2), uu, kPow2C1);
                    em1 = __builtin_fabsf(uu) < 0.0625f ? uu * p : em1;
                }
                ci[j] = em1;
                cd[j] = em1;
                if constexpr (MODE == 2) {
                    ci[j] = zero[j] ? dt : em1;
                    cd[j] = zero[j] ? 0.0f : em1;
                }
            }
        };
        coefs(kT - 1, cin, cdec);
#pragma unroll
        for (int k = kT - 1; k >= 0; --k) {
            float nin[4], ndec[4];
            if (k > 0) coefs(k - 1, nin, ndec);
            const float xt = row_step<T>(xrow, k);
            const float4 bv = *reinterpret_cast<const float4 *>(Bq + k * kNP);
            const float bj[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (MODE == 0) {
                    // cdec holds Ā itself here: R·(Ā − 1)·B x as (R·Ā − R)·B x, one instruction fewer
                    const float rn = R[j] * cdec[j];
                    Eacc[j] = __builtin_fmaf(rn - R[j], bj[j] * xt, Eacc[j]);
                    R[j] = rn;
                } else {
                    Eacc[j] = __builtin_fmaf(R[j] * cin[j], bj[j] * xt, Eacc[j]);
                    R[j] = __builtin_fmaf(R[j], cdec[j], R[j]);
                }
            }
            if (k > 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) { cin[j] = nin[j]; cdec[j] = ndec[j]; }
            }
            // one step per stretch: the next step's exponentials and this step's accumulation interleave
            // here, and nothing of later steps is pulled ahead (which would hold a tile of values at once)
            asm volatile("" : "+v"(cin[0]), "+v"(cin[1]), "+v"(cin[2]), "+v"(cin[3]), "+v"(R[0]), "+v"(R[1]),
                              "+v"(R[2]), "+v"(R[3]));
        }
    };

    float dsum = 0.0f;
    // tiles [it_lo, ntiles) belong to the later part of a split walk, [0, it_lo) to the earlier part
    const int it_lo = ntiles > a.split_tiles ? ntiles - a.split_tiles : 0;
    int it = ntiles - 1;
    if (part == 1) {
        // the earlier part: ΣΔ over the later part's tiles (Δ alone), so that R starts as the decay from the
        // segment end back to it, exp(A·ΣΔ); then the walk continues below it as a whole walk would
        load_tile(t_begin + (int64_t)(ntiles - 1) * kT, false);
#pragma unroll 1
        for (int k = ntiles - 1; k >= it_lo; --k) {  // one tile ahead
            wave_sync();
            store_tile(false);
            wave_sync();
            if (k > it_lo) load_tile(t_begin + (int64_t)(k - 1) * kT, false);
            dsum += row_dsum();
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) R[j] = zero[j] ? 1.0f : exp2_fast(a2[j] * dsum);
        it = it_lo - 1;
    }
    // the walk over tiles [lo, it]: everything for a whole walk, the later part's tiles, or from below them
    const int lo = part == 2 ? it_lo : 0;
    bool walk = it >= lo;
    if (walk && part == 1) {
        bool done = true;
#pragma unroll
        for (int j = 0; j < 4; ++j) done = done && (!live[j] || R[j] <= kStopRel);
        walk = !__all(done);
    }
    if (walk) {
        const int64_t t_last = t_begin + (int64_t)it * kT;
        for (int i = lane; i < kT * kNP; i += kWave) Bs[i] = 0.0f;
        load_tile(t_last, true);
        wave_sync();
        store_tile(true);
        if (it > lo) load_tile(t_last - kT, true);
        wave_sync();
#pragma unroll 1
        for (; it >= lo; --it) {
            const float ts = row_dsum();
            dsum += ts;
            if (wave_zero) {
                walk_tile(std::integral_constant<int, 2>{});
            } else if (__any(ts < thr_sum)) {
                walk_tile(std::integral_constant<int, 1>{});
            } else {
                walk_tile(std::integral_constant<int, 0>{});
            }
            if (it == lo) {
                --it;
                break;
            }
            // stop once every live state's decay back to here is negligible (a NaN never passes)
            bool done = true;
#pragma unroll
            for (int j = 0; j < 4; ++j) done = done && (!live[j] || R[j] <= kStopRel);
            if (__all(done)) {
                --it;
                break;
            }
            const int64_t t0 = t_begin + (int64_t)it * kT;
            wave_sync();  // the walk's reads of the tile come before it is overwritten
            store_tile(true);
            wave_sync();
            if (it > lo + 1) load_tile(t0 - 2 * kT, true);
        }
    }
    // `it` is now the highest tile not walked (−1 when the walk reached the segment start)

    const int64_t base = (seg * a.b * a.d + bi * a.d + ch) * a.N;
    if (part != 2) {
        // P of this wavefront's states. A walk that reached the segment start has summed Δ over all of it, so
        // P = exp(A·ΣΔ) is exact. A walk that stopped at step t_s did so with R ≤ 2^-24 for every live state, and
        // the carried-in state h_in reaches the segment end as P·h_in = R·g(t_s), g(t_s) being h_in carried to
        // t_s without inputs: at most 2^-24·|g(t_s)|, no more than one fp32 rounding of a state at t_s, so P is
        // taken as 0 there and the tiles not walked are never read.
        const bool whole = it < 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (live[j]) a.P[base + n0 + j] = zero[j] ? 1.0f : (whole ? exp2_fast(a2[j] * dsum) : 0.0f);
    }
    float *Eo = part == 1 ? a.E2 : a.E;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (live[j]) Eo[base + n0 + j] = Eacc[j] * isc[j];
}

}  // namespace

hipError_t launch_agg_rev(const AggLaunch &p, hipStream_t stream) {
    if (p.n_seg <= 1) return hipSuccess;
    if (p.N < 1 || p.N > 64) return hipErrorInvalidValue;
    AggArgs a{};
    a.x = p.x; a.delta = p.delta; a.A = p.A; a.B = p.B; a.P = p.P; a.E = p.E; a.E2 = p.E2;
    a.b = p.b; a.d = p.d; a.L = p.L; a.N = p.N; a.seg_len = p.seg_len;
    a.n_cb = (p.d + kWave - 1) / kWave;
    a.n_units = (int64_t)(p.n_seg - 1) * p.b * a.n_cb;
    a.n_grp = (int)((p.N + 3) / 4);
    const int64_t esize = p.bf16 ? 2 : 4;
    auto aligned16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
    a.vec_rows = ((p.L * esize) % 16 == 0) && aligned16(p.x) && aligned16(p.delta);
    a.vec_bc = ((p.L * p.N * esize) % 16 == 0) && aligned16(p.B);
    // the split walk: group 0's later part takes the last eighth of each segment (the fastest fraction
    // measured on the long-context recipe, among 1/3 .. 1/24)
    const int kt = p.bf16 ? 32 : 16;
    a.split_tiles = a.E2 ? (int)((p.seg_len / kt + 7) / 8) : 0;
    const int64_t grid = (a.n_units + kXcds - 1) / kXcds * kXcds * (a.n_grp + (a.E2 ? 1 : 0));
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 g((unsigned)grid), w(kWave);
    if (p.bf16) {
        if (p.N <= 16) hipLaunchKernelGGL((agg_rev_kernel<uint16_t, 16>), g, w, 0, stream, a);
        else hipLaunchKernelGGL((agg_rev_kernel<uint16_t, 64>), g, w, 0, stream, a);
    } else {
        if (p.N <= 16) hipLaunchKernelGGL((agg_rev_kernel<float, 16>), g, w, 0, stream, a);
        else hipLaunchKernelGGL((agg_rev_kernel<float, 64>), g, w, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace ssm
