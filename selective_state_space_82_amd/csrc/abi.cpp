// abi.cpp — the C ABI of libssmscan.so: argument validation, launch planning, scratch, dispatch.
// See include/ssm_scan.h for the contract of every entry point.
#include "ssm_scan.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace {

using ssm::FwdLaunch;
using ssm::StepLaunch;

bool valid_dtype(ssm_dtype_t t) { return t == SSM_F32 || t == SSM_BF16; }

// a * b without overflow past 2^62 (sizes are far below that in practice)
bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > (INT64_C(1) << 62) / a) return false;
    *out = a * b;
    return true;
}

struct Span {
    const void *p;
    int64_t bytes;
};

bool overlaps(const Span &u, const Span &v) {
    if (!u.p || !v.p || u.bytes <= 0 || v.bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(u.p), a1 = a0 + (uintptr_t)u.bytes;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(v.p), b1 = b0 + (uintptr_t)v.bytes;
    return a0 < b1 && b0 < a1;
}

// Compute units of the current device, cached per device id.
int cu_count() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// Stream-ordered scratch comes from a memory pool the library creates on each device at first use. Its
// release threshold is at the maximum, so freed scratch stays in that pool across synchronisations and
// repeated calls do not pay for re-mapping it. The device's default pool is left as the caller set it.
// Should the pool not be created, scratch comes from the default pool as it stands.
hipMemPool_t scratch_pool() {
    static std::mutex mu;
    static hipMemPool_t pools[64] = {};
    static bool tried[64] = {false};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!tried[dev]) {
        tried[dev] = true;
        hipMemPoolProps props{};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) == hipSuccess && pool) {
            uint64_t threshold = UINT64_MAX;
            (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &threshold);
            pools[dev] = pool;
        }
    }
    return pools[dev];
}

hipError_t scratch_alloc(void **p, size_t bytes, hipStream_t stream) {
    hipMemPool_t pool = scratch_pool();
    if (pool) return hipMallocFromPoolAsync(p, bytes, pool, stream);
    return hipMallocAsync(p, bytes, stream);
}

struct Plan {
    int lanes, npl, n_seg;
    int64_t seg_len, waves_per_seg, groups_out, groups_agg, scratch_bytes;
};

// Smallest supported states-per-lane count holding ceil(N / lanes) states (0 = none).
int states_per_lane(int64_t N, int lanes) {
    const int64_t need = (N + lanes - 1) / lanes;
    for (int npl : {4, 8, 16})
        if (need <= npl) return npl;
    return 0;
}

// Launch plan. A workgroup is one wavefront: 64 / G channels of one batch row (G lanes per
// channel, each holding states_per_lane states) over one time segment. A sequence is cut into
// segments only when the channel blocks alone cannot fill the device, since every segment after
// the first costs an aggregate rescan of its inputs.
ssm_status_t make_plan(int64_t b, int64_t d, int64_t L, int64_t N, const ssm_fwd_opts_t *o, int cus, Plan *pl) {
    int lanes = o ? o->lanes_per_channel : 0;
    if (lanes == 0) lanes = 4;
    if (lanes != 1 && lanes != 2 && lanes != 4) return SSM_ERR_UNSUPPORTED;
    const int npl = states_per_lane(N, lanes);
    if (npl == 0) return SSM_ERR_UNSUPPORTED;
    const int64_t cw = 64 / lanes;
    const int64_t ncb = b * ((d + cw - 1) / cw);  // wavefronts per time segment
    int64_t seg_len = o ? o->seg_len : 0;
    if (seg_len < 0 || (seg_len % ssm::kSegQuantum) != 0) return SSM_ERR_UNSUPPORTED;
    const int64_t Lr = ((L + ssm::kSegQuantum - 1) / ssm::kSegQuantum) * ssm::kSegQuantum;
    if (seg_len == 0) {
        // A split in time adds an aggregate pass over (S-1)/S of the sequence (about half the
        // cost of the output pass), so it only pays when one segment gives fewer wavefronts than
        // the chip has SIMDs (4 per compute unit). Then aim at about eight wavefronts per SIMD
        // over the grid, with segments of at least 256 steps.
        const int64_t simds = (int64_t)cus * 4;
        int64_t S = ncb >= simds ? 1 : (simds * 8 + ncb - 1) / ncb;
        const int64_t max_seg = Lr / 256 > 0 ? Lr / 256 : 1;
        if (S > max_seg) S = max_seg;
        if (S > 64) S = 64;
        if (S < 1) S = 1;
        seg_len = ((Lr / S + ssm::kSegQuantum - 1) / ssm::kSegQuantum) * ssm::kSegQuantum;
        // Segments of kAggWalkMinSeg steps or more take the truncated backward aggregate walk, which costs
        // about one walk over the slow states' decay horizon per segment rather than (S-1)/S of the
        // sequence, so fewer, longer segments pay there: aim at about 5.6 wavefronts per SIMD (45/8). On
        // b 1, d 2048, L 131072 (S = 45) a sweep put the output pass at its fastest there, and the
        // aggregate pass no longer shrank below about 47 segments.
        if (S > 1 && seg_len >= ssm::kAggWalkMinSeg) {
            int64_t Sw = (simds * 45 + 8 * ncb - 1) / (8 * ncb);
            if (Sw > S) Sw = S;
            if (Sw < 2) Sw = 2;
            const int64_t sl = (((Lr + Sw - 1) / Sw + ssm::kSegQuantum - 1) / ssm::kSegQuantum) * ssm::kSegQuantum;
            if (sl >= ssm::kAggWalkMinSeg) seg_len = sl;
        }
    }
    if (seg_len > Lr || seg_len == 0) seg_len = Lr > 0 ? Lr : ssm::kSegQuantum;
    int64_t n_seg = L > 0 ? (L + seg_len - 1) / seg_len : 1;
    if (n_seg > 4096) return SSM_ERR_UNSUPPORTED;
    int64_t scratch = 0;
    if (n_seg > 1) {
        int64_t per = 0;
        if (!mul_ok((n_seg - 1) * b, d * N, &per) || !mul_ok(per, 3 * (int64_t)sizeof(float), &scratch))
            return SSM_ERR_SHAPE;
        scratch = ssm::scratch_floats(n_seg, b, d, N) * (int64_t)sizeof(float);
    }
    pl->lanes = lanes;
    pl->npl = npl;
    pl->n_seg = (int)n_seg;
    pl->seg_len = seg_len;
    pl->waves_per_seg = ncb;
    pl->groups_out = n_seg * ncb;
    pl->groups_agg = (n_seg - 1) * ncb;
    pl->scratch_bytes = scratch;
    if (pl->groups_out > 0x7fffffffLL) return SSM_ERR_SHAPE;
    return SSM_OK;
}

// A short sequence on few channel blocks (ssm::small_problem) runs the small-problem kernel, unless an option
// asked for a plan of the main kernel. Its plan: segments of 8 or 16 steps, a workgroup per block of 16 channels
// with a wavefront per segment, no aggregate pass and no scratch.
bool plan_small(int64_t b, int64_t d, int64_t L, int64_t N, const ssm_fwd_opts_t *o, Plan *pl) {
    if (o && (o->seg_len != 0 || o->lanes_per_channel != 0)) return false;
    if (!ssm::small_problem(b, d, L, N)) return false;
    const int64_t ncb = b * ((d + ssm::kSmallCh - 1) / ssm::kSmallCh);
    pl->lanes = 4;
    pl->npl = 4;
    pl->seg_len = ssm::small_seg(L);
    pl->n_seg = (int)((L + pl->seg_len - 1) / pl->seg_len);
    pl->waves_per_seg = ncb;
    pl->groups_out = ncb;
    pl->groups_agg = 0;
    pl->scratch_bytes = 0;
    return true;
}

ssm_status_t check_fwd_sizes(int64_t b, int64_t d, int64_t L, int64_t N, ssm_dtype_t dtype) {
    if (!valid_dtype(dtype)) return SSM_ERR_UNSUPPORTED;
    if (b < 1 || d < 1 || N < 1 || L < 0) return SSM_ERR_SHAPE;
    if (N > SSM_MAX_N) return SSM_ERR_UNSUPPORTED;
    int64_t t = 0;
    if (!mul_ok(b, d, &t) || !mul_ok(t, L > 0 ? L : 1, &t) || !mul_ok(t, N, &t)) return SSM_ERR_SHAPE;
    return SSM_OK;
}

// Option values that need no device information.
ssm_status_t check_opts(int64_t N, const ssm_fwd_opts_t *o) {
    if (!o) return SSM_OK;
    const int lanes = o->lanes_per_channel;
    if (lanes != 0 && lanes != 1 && lanes != 2 && lanes != 4) return SSM_ERR_UNSUPPORTED;
    if (states_per_lane(N, lanes == 0 ? 4 : lanes) == 0) return SSM_ERR_UNSUPPORTED;
    if (o->seg_len < 0 || (o->seg_len % ssm::kSegQuantum) != 0) return SSM_ERR_UNSUPPORTED;
    return SSM_OK;
}

// The fused front end of ssm_scan_fwd_conv / ssm_scan_step_conv (conv_w == nullptr: none).
struct FrontEnd {
    const float *conv_w, *conv_bias, *conv_state_in, *delta_bias;
    float *conv_state_out;
    void *x_out;
    int64_t W;
    int softplus;
};

ssm_status_t fwd_impl(const void *x, const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, void *y, float *final_state, int64_t b, int64_t d,
                      int64_t L, int64_t N, ssm_dtype_t dtype, hipStream_t stream, const ssm_fwd_opts_t *o,
                      bool noalloc = false, const FrontEnd *fe = nullptr) {
    ssm_status_t st = check_fwd_sizes(b, d, L, N, dtype);
    if (st != SSM_OK) return st;
    if (fe) {
        if (fe->W < 1 || fe->W > SSM_MAX_FUSED_CONV_W) return SSM_ERR_UNSUPPORTED;
        if (!fe->conv_w) return SSM_ERR_NULL;
        const int64_t es = dtype == SSM_BF16 ? 2 : 4;
        const int64_t bdl = b * d * L, bdn = b * d * N, bdh = b * d * (fe->W - 1);
        const Span outs[] = {{y, bdl * es}, {final_state, bdn * 4}, {fe->x_out, bdl * es}, {fe->conv_state_out, bdh * 4}};
        const Span ins[] = {{x, bdl * es}, {delta, bdl * es}, {z, bdl * es}, {B, b * L * N * es}, {C, b * L * N * es},
                            {A, d * N * 4}, {D, d * 4}, {o ? o->initial_state : nullptr, bdn * 4},
                            {fe->conv_w, d * fe->W * 4}, {fe->conv_bias, d * 4}, {fe->conv_state_in, bdh * 4},
                            {fe->delta_bias, d * 4}};
        for (size_t i = 0; i < 4; ++i) {
            for (const Span &s : ins)
                if (overlaps(outs[i], s)) return SSM_ERR_ALIAS;
            for (size_t j = i + 1; j < 4; ++j)
                if (overlaps(outs[i], outs[j])) return SSM_ERR_ALIAS;
        }
        if (L == 0 && fe->conv_state_out && fe->W > 1) {  // the state passes through unchanged
            const hipError_t e = fe->conv_state_in
                ? hipMemcpyAsync(fe->conv_state_out, fe->conv_state_in, (size_t)bdh * 4, hipMemcpyDeviceToDevice, stream)
                : ssm::launch_fill_zero(fe->conv_state_out, bdh, stream);
            if (e != hipSuccess) return SSM_ERR_HIP;
        }
    }
    // With L = 0 nothing but final_state is touched, so the (empty) sequence tensors may be NULL.
    if (L > 0 && (!x || !delta || !A || !B || !C || !y)) return SSM_ERR_NULL;
    st = check_opts(N, o);
    if (st != SSM_OK) return st;
    const int64_t es = dtype == SSM_BF16 ? 2 : 4;
    const int64_t bdl = b * d * L, bln = b * L * N, bdn = b * d * N;
    const Span sy{y, bdl * es}, sf{final_state, bdn * 4};
    const Span ins[] = {{x, bdl * es}, {delta, bdl * es}, {z, bdl * es}, {B, bln * es}, {C, bln * es},
                        {A, d * N * 4}, {D, d * 4}, {o ? o->initial_state : nullptr, bdn * 4}};
    for (const Span &s : ins)
        if (overlaps(sy, s) || overlaps(sf, s)) return SSM_ERR_ALIAS;
    if (overlaps(sy, sf)) return SSM_ERR_ALIAS;

    if (L == 0) {  // the state passes through: the initial state, or zeros
        const float *h0 = o ? o->initial_state : nullptr;
        if (final_state) {
            const hipError_t e = h0 ? hipMemcpyAsync(final_state, h0, (size_t)bdn * 4, hipMemcpyDeviceToDevice, stream)
                                    : ssm::launch_fill_zero(final_state, bdn, stream);
            if (e != hipSuccess) return SSM_ERR_HIP;
        }
        return SSM_OK;
    }
    Plan pl{};
    st = make_plan(b, d, L, N, o, cu_count(), &pl);
    if (st != SSM_OK) return st;
    FwdLaunch p{};
    p.small = !fe && plan_small(b, d, L, N, o, &pl);
    p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.y = y;
    p.final_state = final_state;
    p.init_state = o ? o->initial_state : nullptr;
    p.b = b; p.d = d; p.L = L; p.N = N;
    p.bf16 = dtype == SSM_BF16;
    p.lanes_per_channel = pl.lanes;
    p.states_per_lane = pl.npl;
    p.seg_len = pl.seg_len;
    p.n_seg = pl.n_seg;
    p.ev_begin = o ? static_cast<hipEvent_t>(o->ev_begin) : nullptr;
    p.ev_end = o ? static_cast<hipEvent_t>(o->ev_end) : nullptr;
    if (fe) {
        p.conv_w = fe->conv_w; p.conv_bias = fe->conv_bias; p.conv_state_in = fe->conv_state_in;
        p.conv_state_out = fe->W > 1 ? fe->conv_state_out : nullptr; p.x_out = fe->x_out;
        p.delta_bias = fe->delta_bias; p.conv_W = (int)fe->W; p.delta_softplus = fe->softplus ? 1 : 0;
    }
    void *scratch = nullptr;
    if (noalloc) {
        // the fixed device array: nothing allocated, nothing to clear (every scratch word a call reads
        // is written earlier in the same call)
        if (pl.scratch_bytes > ssm::kNoAllocScratchBytes) return SSM_ERR_SCRATCH;
        if (pl.scratch_bytes > 0 && ssm::noalloc_scratch(&p.scratch) != hipSuccess) return SSM_ERR_HIP;
        return ssm::launch_scan_fwd(p, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
    }
    if (pl.scratch_bytes > 0) {
        if (scratch_alloc(&scratch, (size_t)pl.scratch_bytes, stream) != hipSuccess) return SSM_ERR_HIP;
        p.scratch = static_cast<float *>(scratch);
    }
    const hipError_t e = ssm::launch_scan_fwd(p, stream);
    if (scratch) {
        if (hipFreeAsync(scratch, stream) != hipSuccess) return SSM_ERR_HIP;
    }
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

// Time split of the reverse aggregate and gradient passes, as a segment length. The gradient kernel
// keeps two wavefronts per SIMD resident at 4 states per lane and one above that (its registers and
// LDS), so its grid runs in rounds of that many wavefronts, and a partial last round leaves SIMDs idle.
// The split minimises rounds × segment length; a longer split wins only where it saves more than
// 1/16 of that, since every segment after the first costs a reverse aggregate rescan.
int64_t grad_seg_len(int64_t b, int64_t d, int64_t L, int lanes, int npl, int cus) {
    const int64_t q = ssm::kSegQuantum;
    const int64_t Lr = ((L + q - 1) / q) * q;
    const int64_t ncb = b * ((d + 64 / lanes - 1) / (64 / lanes));
    const int64_t resident = (int64_t)cus * 4 * (npl <= 4 ? 2 : 1);
    int64_t best_len = Lr, best_cost = 0;
    const int64_t max_seg = Lr / 128 > 1 ? (Lr / 128 < 64 ? Lr / 128 : 64) : 1;
    for (int64_t S = 1; S <= max_seg; ++S) {
        const int64_t len = ((Lr / S + q - 1) / q) * q;
        const int64_t segs = (L + len - 1) / len;
        const int64_t rounds = (segs * ncb + resident - 1) / resident;
        const int64_t cost = rounds * len;
        if (S == 1 || cost * 16 < best_cost * 15) {
            best_cost = cost;
            best_len = len;
        }
    }
    return best_len;
}

ssm_status_t bwd_impl(const void *x, const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *initial_state, const void *dy,
                      const float *d_final_state, void *dx, void *ddelta, float *dA, float *dB, float *dC,
                      float *dD, void *dz, float *d_initial_state, int64_t b, int64_t d, int64_t L, int64_t N,
                      ssm_dtype_t dtype, hipStream_t stream) {
    ssm_status_t st = check_fwd_sizes(b, d, L, N, dtype);
    if (st != SSM_OK) return st;
    if (L < 1) return SSM_ERR_SHAPE;
    if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC) return SSM_ERR_NULL;
    if (z && !dz) return SSM_ERR_NULL;
    if (!z) dz = nullptr;
    const int64_t es = dtype == SSM_BF16 ? 2 : 4;
    const int64_t bdl = b * d * L, bln = b * L * N, bdn = b * d * N;
    const Span outs[] = {{dx, bdl * es}, {ddelta, bdl * es}, {dz, bdl * es}, {dA, d * N * 4},
                         {dB, bln * 4}, {dC, bln * 4}, {dD, d * 4}, {d_initial_state, bdn * 4}};
    const Span ins[] = {{x, bdl * es}, {delta, bdl * es}, {z, bdl * es}, {B, bln * es}, {C, bln * es},
                        {A, d * N * 4}, {D, d * 4}, {initial_state, bdn * 4}, {dy, bdl * es},
                        {d_final_state, bdn * 4}};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Span &s : ins)
            if (overlaps(outs[i], s)) return SSM_ERR_ALIAS;
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlaps(outs[i], outs[j])) return SSM_ERR_ALIAS;
    }
    Plan pl{};
    st = make_plan(b, d, L, N, nullptr, cu_count(), &pl);
    if (st != SSM_OK) return st;
    ssm::BwdLaunch p{};
    p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.init_state = initial_state;
    p.dy = dy; p.d_final_state = d_final_state; p.dx = dx; p.ddelta = ddelta; p.dz = dz;
    p.dA = dA; p.dB = dB; p.dC = dC; p.dD = dD; p.d_init_state = d_initial_state;
    p.b = b; p.d = d; p.L = L; p.N = N; p.bf16 = dtype == SSM_BF16;
    p.lanes_per_channel = pl.lanes; p.states_per_lane = pl.npl; p.seg_len = pl.seg_len; p.n_seg = pl.n_seg;
    p.grad_seg_len = grad_seg_len(b, d, L, pl.lanes, pl.npl, cu_count());
    p.grad_n_seg = (int)((L + p.grad_seg_len - 1) / p.grad_seg_len);
    int64_t floats = 0;
    if (!mul_ok(b * d, L, &floats)) return SSM_ERR_SHAPE;
    floats = ssm::bwd_scratch_floats(pl.n_seg, p.grad_n_seg, b, d, L, N, pl.npl);
    void *scratch = nullptr;
    if (scratch_alloc(&scratch, (size_t)floats * sizeof(float), stream) != hipSuccess) return SSM_ERR_HIP;
    p.scratch = static_cast<float *>(scratch);
    const hipError_t e = ssm::launch_scan_bwd(p, stream);
    if (hipFreeAsync(scratch, stream) != hipSuccess) return SSM_ERR_HIP;
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t lti_kernel_check(const float *delta, const float *A, const float *B, const float *C, const float *K,
                              int64_t d, int64_t L, int64_t N) {
    if (d < 1 || N < 1 || L < 0 || L >= (INT64_C(1) << 24)) return SSM_ERR_SHAPE;
    if (N > SSM_MAX_N) return SSM_ERR_UNSUPPORTED;
    int64_t dn = 0, dl = 0;
    if (!mul_ok(d, N, &dn) || !mul_ok(d, L, &dl) || !mul_ok(dl, 4, &dl)) return SSM_ERR_SHAPE;
    if (!delta || !A || !B || !C || (L > 0 && !K)) return SSM_ERR_NULL;
    const Span out{K, dl};
    const Span ins[] = {{delta, d * 4}, {A, dn * 4}, {B, dn * 4}, {C, dn * 4}};
    for (const Span &in : ins)
        if (overlaps(out, in)) return SSM_ERR_ALIAS;
    return SSM_OK;
}

// K == nullptr is accepted only when the caller computes K itself (internal).
ssm_status_t lti_conv_check(const void *x, const float *K, bool k_internal, const float *D, const void *z,
                            const void *y, int64_t b, int64_t d, int64_t L, ssm_dtype_t dtype) {
    if (!valid_dtype(dtype)) return SSM_ERR_UNSUPPORTED;
    if (b < 1 || d < 1 || d > (INT64_C(1) << 22) || L < 1) return SSM_ERR_SHAPE;
    if (L > SSM_LTI_MAX_L && !k_internal) return SSM_ERR_UNSUPPORTED;  // one transform holds a given K
    if (L >= (INT64_C(1) << 40)) return SSM_ERR_SHAPE;
    int64_t bdl = 0;
    if (!mul_ok(b, d, &bdl) || !mul_ok(bdl, L, &bdl)) return SSM_ERR_SHAPE;
    if (!x || (!K && !k_internal) || !y) return SSM_ERR_NULL;
    const int64_t es = dtype == SSM_BF16 ? 2 : 4;
    const Span out{y, bdl * es};
    const Span ins[] = {{x, bdl * es}, {z, bdl * es}, {K, K ? d * L * 4 : 0}, {D, d * 4}};
    for (const Span &in : ins)
        if (overlaps(out, in)) return SSM_ERR_ALIAS;
    return SSM_OK;
}

}  // namespace

extern "C" {

const char *ssm_status_string(ssm_status_t s) {
    switch (s) {
        case SSM_OK: return "SSM_OK";
        case SSM_ERR_NULL: return "SSM_ERR_NULL: a required pointer is NULL";
        case SSM_ERR_SHAPE: return "SSM_ERR_SHAPE: a size is out of range";
        case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED: N, dtype or an option value is not supported";
        case SSM_ERR_HIP: return "SSM_ERR_HIP: a HIP runtime call or kernel launch failed";
        case SSM_ERR_ALIAS: return "SSM_ERR_ALIAS: an output overlaps an input or another output";
        case SSM_STATUS_MAX_ENUM: break;
        case SSM_ERR_SCRATCH:
            return "SSM_ERR_SCRATCH: the call needs more scratch than ssm_scan_fwd_noalloc holds "
                   "(SSM_NOALLOC_SCRATCH_BYTES); use fewer time segments or ssm_scan_fwd_ex";
    }
    return "unknown ssm_status_t";
}

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

ssm_status_t ssm_scan_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C,
                          const float *D, const void *z, void *y, float *final_state, int64_t b, int64_t d,
                          int64_t L, int64_t N, ssm_dtype_t dtype, hipStream_t stream) {
    return fwd_impl(x, delta, A, B, C, D, z, y, final_state, b, d, L, N, dtype, stream, nullptr);
}

ssm_status_t ssm_scan_fwd_ex(const void *x, const void *delta, const float *A, const void *B, const void *C,
                             const float *D, const void *z, void *y, float *final_state, int64_t b, int64_t d,
                             int64_t L, int64_t N, ssm_dtype_t dtype, hipStream_t stream,
                             const ssm_fwd_opts_t *opts) {
    return fwd_impl(x, delta, A, B, C, D, z, y, final_state, b, d, L, N, dtype, stream, opts);
}

ssm_status_t ssm_scan_fwd_noalloc(const void *x, const void *delta, const float *A, const void *B, const void *C,
                                  const float *D, const void *z, void *y, float *final_state, int64_t b, int64_t d,
                                  int64_t L, int64_t N, ssm_dtype_t dtype, hipStream_t stream,
                                  const ssm_fwd_opts_t *opts) {
    return fwd_impl(x, delta, A, B, C, D, z, y, final_state, b, d, L, N, dtype, stream, opts, true);
}

ssm_status_t ssm_scan_fwd_conv(const void *xin, const float *conv_w, const float *conv_bias, const float *conv_state_in,
                               int64_t W, const void *delta, const float *delta_bias, int32_t delta_softplus,
                               const float *A, const void *B, const void *C, const float *D, const void *z,
                               const float *initial_state, void *y, float *final_state, float *conv_state_out,
                               void *x_out, int64_t b, int64_t d, int64_t L, int64_t N, ssm_dtype_t dtype,
                               hipStream_t stream) {
    const FrontEnd fe{conv_w, conv_bias, conv_state_in, delta_bias, conv_state_out, x_out, W, delta_softplus};
    ssm_fwd_opts_t o{};
    o.initial_state = initial_state;
    return fwd_impl(xin, delta, A, B, C, D, z, y, final_state, b, d, L, N, dtype, stream, &o, false, &fe);
}

ssm_status_t ssm_scan_step_conv(float *state, float *conv_state, const void *xin, const float *conv_w,
                                const float *conv_bias, int64_t W, const void *delta, const float *delta_bias,
                                int32_t delta_softplus, const float *A, const void *B, const void *C, const float *D,
                                const void *z, void *y, void *x_out, int64_t b, int64_t d, int64_t N,
                                ssm_dtype_t dtype, hipStream_t stream) {
    if (!state || !xin || !delta || !A || !B || !C || !y || !conv_w || (W > 1 && !conv_state)) return SSM_ERR_NULL;
    if (!valid_dtype(dtype)) return SSM_ERR_UNSUPPORTED;
    if (b < 1 || d < 1 || N < 1) return SSM_ERR_SHAPE;
    if (N > SSM_MAX_N || W < 1 || W > SSM_MAX_FUSED_CONV_W) return SSM_ERR_UNSUPPORTED;
    int64_t bd = 0, bdn = 0, tmp = 0;
    if (!mul_ok(b, d, &bd) || !mul_ok(bd, N, &bdn) || !mul_ok(bd, 16, &tmp)) return SSM_ERR_SHAPE;
    if (bd > 0x7fffffffLL) return SSM_ERR_SHAPE;
    const int64_t es = dtype == SSM_BF16 ? 2 : 4;
    const Span outs[] = {{y, bd * es}, {state, bdn * 4}, {conv_state, bd * (W - 1) * 4}, {x_out, bd * es}};
    const Span ins[] = {{xin, bd * es}, {delta, bd * es}, {z, bd * es}, {B, b * N * es}, {C, b * N * es},
                        {A, d * N * 4}, {D, d * 4}, {conv_w, d * W * 4}, {conv_bias, d * 4}, {delta_bias, d * 4}};
    for (size_t i = 0; i < 4; ++i) {
        for (const Span &s : ins)
            if (overlaps(outs[i], s)) return SSM_ERR_ALIAS;
        for (size_t j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], outs[j])) return SSM_ERR_ALIAS;
    }
    StepLaunch p{};
    p.state = state; p.x = xin; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.y = y;
    p.b = b; p.d = d; p.N = N; p.bf16 = dtype == SSM_BF16;
    p.conv_state = conv_state; p.conv_w = conv_w; p.conv_bias = conv_bias; p.delta_bias = delta_bias;
    p.x_out = x_out; p.conv_W = (int)W; p.delta_softplus = delta_softplus ? 1 : 0;
    return ssm::launch_scan_step(p, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_scan_fwd_plan(int64_t b, int64_t d, int64_t L, int64_t N, ssm_dtype_t dtype,
                               const ssm_fwd_opts_t *opts, ssm_fwd_plan_t *plan) {
    if (!plan) return SSM_ERR_NULL;
    ssm_status_t st = check_fwd_sizes(b, d, L, N, dtype);
    if (st != SSM_OK) return st;
    st = check_opts(N, opts);
    if (st != SSM_OK) return st;
    Plan pl{};
    st = make_plan(b, d, L, N, opts, 256, &pl);
    if (st != SSM_OK) return st;
    plan_small(b, d, L, N, opts, &pl);
    plan->seg_len = (int32_t)pl.seg_len;
    plan->lanes_per_channel = pl.lanes;
    plan->states_per_lane = pl.npl;
    plan->n_segments = pl.n_seg;
    plan->waves_per_segment = pl.waves_per_seg;
    plan->groups_output_pass = pl.groups_out;
    plan->groups_aggregate_pass = pl.groups_agg;
    plan->scratch_bytes = pl.scratch_bytes;
    return SSM_OK;
}

ssm_status_t ssm_scan_bwd(const void *x, const void *delta, const float *A, const void *B, const void *C,
                          const float *D, const void *z, const float *initial_state, const void *dy,
                          const float *d_final_state, void *dx, void *ddelta, float *dA, float *dB, float *dC,
                          float *dD, void *dz, float *d_initial_state, int64_t b, int64_t d, int64_t L, int64_t N,
                          ssm_dtype_t dtype, hipStream_t stream) {
    return bwd_impl(x, delta, A, B, C, D, z, initial_state, dy, d_final_state, dx, ddelta, dA, dB, dC, dD, dz,
                    d_initial_state, b, d, L, N, dtype, stream);
}

ssm_status_t ssm_conv1d_fwd(const void *xin, const float *w, const float *bias, const float *state_in, void *x_out,
                            float *state_out, int64_t b, int64_t d, int64_t L, int64_t W, int32_t apply_silu,
                            ssm_dtype_t dtype, hipStream_t stream) {
    if (!valid_dtype(dtype)) return SSM_ERR_UNSUPPORTED;
    if (b < 1 || d < 1 || L < 0 || W < 1) return SSM_ERR_SHAPE;
    if (W > SSM_MAX_CONV_W) return SSM_ERR_UNSUPPORTED;
    int64_t bdl = 0, bd = 0;
    if (!mul_ok(b, d, &bd) || !mul_ok(bd, L > 0 ? L : 1, &bdl) || !mul_ok(bdl, 16, &bdl)) return SSM_ERR_SHAPE;
    bdl /= 16;
    if (!w || (L > 0 && (!xin || !x_out))) return SSM_ERR_NULL;
    const int64_t es = dtype == SSM_BF16 ? 2 : 4;
    const Span so{x_out, bdl * es}, ss{state_out, bd * (W - 1) * 4};
    const Span ins[] = {{xin, bdl * es}, {w, d * W * 4}, {bias, d * 4}};
    for (const Span &s : ins)
        if (overlaps(so, s) || overlaps(ss, s)) return SSM_ERR_ALIAS;
    if (overlaps(so, ss) || overlaps(so, Span{state_in, bd * (W - 1) * 4})) return SSM_ERR_ALIAS;
    if (state_out && state_in && state_out != state_in && overlaps(ss, Span{state_in, bd * (W - 1) * 4}))
        return SSM_ERR_ALIAS;
    ssm::ConvLaunch p{};
    p.xin = xin; p.w = w; p.bias = bias; p.state_in = state_in; p.xout = x_out; p.state_out = state_out;
    p.b = b; p.d = d; p.L = L; p.W = (int)W; p.silu_on = apply_silu ? 1 : 0; p.bf16 = dtype == SSM_BF16;
    return ssm::launch_conv1d(p, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_conv1d_step(float *state, const void *xin, const float *w, const float *bias, void *x_out,
                             int64_t b, int64_t d, int64_t W, int32_t apply_silu, ssm_dtype_t dtype,
                             hipStream_t stream) {
    if (!valid_dtype(dtype)) return SSM_ERR_UNSUPPORTED;
    if (b < 1 || d < 1 || W < 1) return SSM_ERR_SHAPE;
    if (W > SSM_MAX_CONV_W) return SSM_ERR_UNSUPPORTED;
    int64_t bd = 0, tmp = 0;
    if (!mul_ok(b, d, &bd) || !mul_ok(bd, 16 * W, &tmp)) return SSM_ERR_SHAPE;
    if (!xin || !w || !x_out || (W > 1 && !state)) return SSM_ERR_NULL;
    const int64_t es = dtype == SSM_BF16 ? 2 : 4;
    const Span so{x_out, bd * es}, ss{state, bd * (W - 1) * 4};
    const Span ins[] = {{xin, bd * es}, {w, d * W * 4}, {bias, d * 4}};
    for (const Span &s : ins)
        if (overlaps(so, s) || overlaps(ss, s)) return SSM_ERR_ALIAS;
    if (overlaps(so, ss)) return SSM_ERR_ALIAS;
    ssm::ConvStepLaunch p{};
    p.state = state; p.xin = xin; p.w = w; p.bias = bias; p.xout = x_out;
    p.b = b; p.d = d; p.W = (int)W; p.silu_on = apply_silu ? 1 : 0; p.bf16 = dtype == SSM_BF16;
    return ssm::launch_conv_step(p, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_scan_step(float *state, const void *x, const void *delta, const float *A, const void *B,
                           const void *C, const float *D, const void *z, void *y, int64_t b, int64_t d,
                           int64_t N, ssm_dtype_t dtype, hipStream_t stream) {
    if (!state || !x || !delta || !A || !B || !C || !y) return SSM_ERR_NULL;
    if (!valid_dtype(dtype)) return SSM_ERR_UNSUPPORTED;
    if (b < 1 || d < 1 || N < 1) return SSM_ERR_SHAPE;
    if (N > SSM_MAX_N) return SSM_ERR_UNSUPPORTED;
    int64_t bd = 0, bdn = 0, tmp = 0;
    if (!mul_ok(b, d, &bd) || !mul_ok(bd, N, &bdn) || !mul_ok(bd, 16, &tmp)) return SSM_ERR_SHAPE;
    if (bd > 0x7fffffffLL) return SSM_ERR_SHAPE;  // (b, d) pairs are indexed in 32 bits
    const int64_t es = dtype == SSM_BF16 ? 2 : 4;
    const Span sy{y, bd * es}, ss{state, bdn * 4};
    const Span ins[] = {{x, bd * es}, {delta, bd * es}, {z, bd * es}, {B, b * N * es}, {C, b * N * es},
                        {A, d * N * 4}, {D, d * 4}};
    for (const Span &s : ins)
        if (overlaps(sy, s) || overlaps(ss, s)) return SSM_ERR_ALIAS;
    if (overlaps(sy, ss)) return SSM_ERR_ALIAS;
    StepLaunch p{};
    p.state = state; p.x = x; p.delta = delta; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.y = y;
    p.b = b; p.d = d; p.N = N;
    p.bf16 = dtype == SSM_BF16;
    return ssm::launch_scan_step(p, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_lti_kernel(const float *delta, const float *A, const float *B, const float *C, float *K, int64_t d,
                            int64_t L, int64_t N, hipStream_t stream) {
    const ssm_status_t st = lti_kernel_check(delta, A, B, C, K, d, L, N);
    if (st != SSM_OK) return st;
    const ssm::LtiKernelLaunch p{delta, A, B, C, K, d, L, N};
    return ssm::launch_lti_kernel(p, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_lti_conv(const void *x, const float *K, const float *D, const void *z, void *y, int64_t b, int64_t d,
                          int64_t L, ssm_dtype_t dtype, hipStream_t stream) {
    const ssm_status_t st = lti_conv_check(x, K, false, D, z, y, b, d, L, dtype);
    if (st != SSM_OK) return st;
    ssm::LtiConvLaunch p{};
    p.x = x; p.z = z; p.K = K; p.D = D; p.y = y; p.b = b; p.d = d; p.L = L; p.bf16 = dtype == SSM_BF16;
    return ssm::launch_lti_conv(p, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_lti_fwd(const void *x, const float *delta, const float *A, const float *B, const float *C,
                         const float *D, const void *z, void *y, int64_t b, int64_t d, int64_t L, int64_t N,
                         ssm_dtype_t dtype, hipStream_t stream) {
    const ssm_status_t st = lti_conv_check(x, nullptr, true, D, z, y, b, d, L, dtype);
    if (st != SSM_OK) return st;
    if (!delta || !A || !B || !C) return SSM_ERR_NULL;
    if (N < 1) return SSM_ERR_SHAPE;
    if (N > SSM_MAX_N) return SSM_ERR_UNSUPPORTED;
    const int64_t es = dtype == SSM_BF16 ? 2 : 4;
    const Span out{y, b * d * L * es};
    const Span ins[] = {{delta, d * 4}, {A, d * N * 4}, {B, d * N * 4}, {C, d * N * 4}};
    for (const Span &in : ins)
        if (overlaps(out, in)) return SSM_ERR_ALIAS;
    // Up to one transform's length: K̄ over the whole sequence, one convolution. Beyond it, the chunked form:
    // K̄ over one chunk, the states between chunks (each chunk's end state from zero, chained by Ā^chunk),
    // and a convolution per chunk that adds the response of the state entering it.
    const bool chunked = L > SSM_LTI_MAX_L;
    const int64_t klen = chunked ? ssm::kLtiChunk : L;
    const int64_t n_chunks = (L + klen - 1) / klen;
    int64_t hfl = 0;
    if (chunked && (!mul_ok(b * d, (n_chunks - 1) * N, &hfl) || hfl > (INT64_C(1) << 40))) return SSM_ERR_SHAPE;
    void *K = nullptr, *H = nullptr;
    if (scratch_alloc(&K, (size_t)(d * klen) * sizeof(float), stream) != hipSuccess) return SSM_ERR_HIP;
    if (chunked && scratch_alloc(&H, (size_t)hfl * sizeof(float), stream) != hipSuccess) {
        (void)hipFreeAsync(K, stream);
        return SSM_ERR_HIP;
    }
    const ssm::LtiKernelLaunch pk{delta, A, B, C, static_cast<float *>(K), d, klen, N};
    hipError_t e = ssm::launch_lti_kernel(pk, stream);
    if (e == hipSuccess && chunked) {
        const ssm::LtiChunkLaunch ph{x, delta, A, B, static_cast<float *>(H), b, d, L, N, klen, dtype == SSM_BF16};
        e = ssm::launch_lti_chunk_states(ph, stream);
    }
    if (e == hipSuccess) {
        ssm::LtiConvLaunch pc{};
        pc.x = x; pc.z = z; pc.K = static_cast<const float *>(K); pc.D = D; pc.y = y;
        pc.b = b; pc.d = d; pc.L = L; pc.bf16 = dtype == SSM_BF16;
        if (chunked) {
            pc.chunk = klen; pc.h_in = static_cast<const float *>(H); pc.delta = delta; pc.A = A; pc.C = C; pc.N = N;
        }
        e = ssm::launch_lti_conv(pc, stream);
    }
    const hipError_t f1 = hipFreeAsync(K, stream);
    const hipError_t f2 = H ? hipFreeAsync(H, stream) : hipSuccess;
    if (f1 != hipSuccess || f2 != hipSuccess) return SSM_ERR_HIP;
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status_t ssm_ssd_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C,
                         const float *D, const void *z, const float *initial_state, void *y, float *final_state,
                         int64_t b, int64_t H, int64_t P, int64_t L, int64_t N, ssm_dtype_t dtype,
                         hipStream_t stream) {
    if (!valid_dtype(dtype)) return SSM_ERR_UNSUPPORTED;
    if (b < 1 || H < 1 || P < 1 || L < 0 || N < 1) return SSM_ERR_SHAPE;
    if (P != 64 || (N != 32 && N != 64 && N != 128)) return SSM_ERR_UNSUPPORTED;
    int64_t bd = 0, bdl = 0, bhl = 0, bln = 0, bdn = 0;
    if (!mul_ok(b, H * P, &bd) || !mul_ok(bd, L > 0 ? L : 1, &bdl) || !mul_ok(b * H, L > 0 ? L : 1, &bhl) ||
        !mul_ok(b * L, N, &bln) || !mul_ok(bd, N, &bdn) || bdl > (INT64_C(1) << 40))
        return SSM_ERR_SHAPE;
    if (b * H * ((L + 63) / 64) >= (INT64_C(1) << 31)) return SSM_ERR_SHAPE;
    if (L > 0 && (!x || !delta || !A || !B || !C || !y)) return SSM_ERR_NULL;
    const int64_t es = dtype == SSM_BF16 ? 2 : 4;
    const Span outs[] = {{y, bdl * es}, {final_state, bdn * 4}};
    const Span ins[] = {{x, bdl * es}, {delta, bhl * es}, {A, H * 4}, {B, bln * es}, {C, bln * es},
                        {D, H * P * 4}, {z, bdl * es}, {initial_state, bdn * 4}};
    for (const Span &o : outs)
        for (const Span &in : ins)
            if (overlaps(o, in)) return SSM_ERR_ALIAS;
    if (overlaps(outs[0], outs[1])) return SSM_ERR_ALIAS;
    if (L == 0) {
        if (final_state) {
            const hipError_t e = initial_state
                ? hipMemcpyAsync(final_state, initial_state, (size_t)bdn * 4, hipMemcpyDeviceToDevice, stream)
                : ssm::launch_fill_zero(final_state, bdn, stream);
            return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
        }
        return SSM_OK;
    }
    void *scratch = nullptr;
    const int cus = cu_count();
    const int64_t floats = ssm::ssd_scratch_floats(b, H, L, N, dtype == SSM_BF16, cus);
    if (floats > 0) {
        if (scratch_alloc(&scratch, (size_t)floats * sizeof(float), stream) != hipSuccess) return SSM_ERR_HIP;
    }
    ssm::SsdLaunch p{};
    p.x = x; p.delta = delta; p.B = B; p.C = C; p.z = z; p.A = A; p.D = D; p.h0 = initial_state;
    p.y = y; p.hT = final_state; p.scratch = static_cast<float *>(scratch);
    p.b = b; p.H = H; p.L = L; p.N = N; p.bf16 = dtype == SSM_BF16;
    p.cus = cus;
    const hipError_t e = ssm::launch_ssd(p, stream);
    if (scratch && hipFreeAsync(scratch, stream) != hipSuccess) return SSM_ERR_HIP;
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"
