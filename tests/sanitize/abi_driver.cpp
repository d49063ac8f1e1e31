// abi_driver.cpp — runs the C ABI's host paths under the address and undefined-behaviour sanitizers (no GPU):
// argument validation, overflow checks, aliasing, plans, status strings, and calls that pass validation and
// reach the (stubbed) launchers or the scratch allocation. Fake device addresses are never dereferenced.
#include <cstdio>
#include <cstdint>

#include "ssm_scan.h"

namespace ssm {
extern int g_launches;
}

static int failures = 0;

static void expect(ssm_status_t got, ssm_status_t want, const char *what) {
    if (got != want) {
        std::printf("FAIL %s: got %d (%s), want %d\n", what, (int)got, ssm_status_string(got), (int)want);
        ++failures;
    }
}

// distinct, non-overlapping fake device addresses, 256 MiB apart
static void *fake(int k) { return reinterpret_cast<void *>(uintptr_t(0x100000000ull) + uintptr_t(k) * (uintptr_t(1) << 28)); }
static float *ffake(int k) { return static_cast<float *>(fake(k)); }

int main() {
    const ssm_dtype_t F = SSM_F32, H = SSM_BF16;
    void *x = fake(1), *dl = fake(2), *B = fake(3), *C = fake(4), *z = fake(5), *y = fake(6);
    float *A = ffake(7), *D = ffake(8), *h = ffake(9);

    // validation failures: nothing launched
    const int before = ssm::g_launches;
    expect(ssm_scan_fwd(nullptr, dl, A, B, C, D, z, y, h, 1, 4, 16, 4, F, nullptr), SSM_ERR_NULL, "null x");
    expect(ssm_scan_fwd(x, dl, A, B, C, D, z, y, h, 0, 4, 16, 4, F, nullptr), SSM_ERR_SHAPE, "b = 0");
    expect(ssm_scan_fwd(x, dl, A, B, C, D, z, y, h, 1, 4, -1, 4, F, nullptr), SSM_ERR_SHAPE, "L < 0");
    expect(ssm_scan_fwd(x, dl, A, B, C, D, z, y, h, 1, 4, 16, 65, F, nullptr), SSM_ERR_UNSUPPORTED, "N > 64");
    expect(ssm_scan_fwd(x, dl, A, B, C, D, z, y, h, 1, 4, 16, 4, (ssm_dtype_t)7, nullptr), SSM_ERR_UNSUPPORTED, "dtype");
    expect(ssm_scan_fwd(x, dl, A, B, C, D, z, y, h, INT64_C(1) << 40, INT64_C(1) << 40, 16, 4, F, nullptr),
           SSM_ERR_SHAPE, "b * d overflow");
    expect(ssm_scan_fwd(x, dl, A, B, C, D, z, x, h, 1, 4, 16, 4, F, nullptr), SSM_ERR_ALIAS, "y aliases x");
    expect(ssm_scan_fwd(x, dl, A, B, C, D, z, y, reinterpret_cast<float *>(static_cast<char *>(y) + 8), 1, 4, 16, 4,
                        F, nullptr),
           SSM_ERR_ALIAS, "final state overlaps y");
    ssm_fwd_opts_t o{};
    o.seg_len = 33;
    expect(ssm_scan_fwd_ex(x, dl, A, B, C, D, z, y, h, 1, 4, 64, 4, F, nullptr, &o), SSM_ERR_UNSUPPORTED, "seg_len");
    o.seg_len = 0;
    o.lanes_per_channel = 3;
    expect(ssm_scan_fwd_ex(x, dl, A, B, C, D, z, y, h, 1, 4, 64, 4, F, nullptr, &o), SSM_ERR_UNSUPPORTED, "lanes");
    expect(ssm_scan_step(nullptr, x, dl, A, B, C, D, z, y, 2, 4, 16, H, nullptr), SSM_ERR_NULL, "step null state");
    expect(ssm_scan_step(h, x, dl, A, B, C, D, z, y, INT64_C(1) << 20, INT64_C(1) << 12, 16, H, nullptr), SSM_ERR_SHAPE,
           "step b * d >= 2^31");
    expect(ssm_conv1d_fwd(x, A, D, nullptr, y, h, 1, 4, 16, 9, 1, F, nullptr), SSM_ERR_UNSUPPORTED, "conv W > 8");
    expect(ssm_scan_fwd_conv(x, A, D, nullptr, 5, dl, nullptr, 1, A, B, C, D, z, nullptr, y, h, nullptr, nullptr, 1, 4,
                             16, 4, F, nullptr),
           SSM_ERR_UNSUPPORTED, "fused W > 4");
    expect(ssm_scan_fwd_conv(x, nullptr, D, nullptr, 4, dl, nullptr, 1, A, B, C, D, z, nullptr, y, h, nullptr, nullptr,
                             1, 4, 16, 4, F, nullptr),
           SSM_ERR_NULL, "fused null taps");
    float *cs = ffake(10);
    expect(ssm_scan_fwd_conv(x, A, D, cs, 4, dl, nullptr, 1, A, B, C, D, z, nullptr, y, h, cs, nullptr, 1, 4, 16, 4, F,
                             nullptr),
           SSM_ERR_ALIAS, "fused Conv1D state in place");
    expect(ssm_lti_conv(x, A, D, z, y, 1, 4, SSM_LTI_MAX_L + 1, F, nullptr), SSM_ERR_UNSUPPORTED, "lti long L");
    expect(ssm_ssd_fwd(x, dl, A, B, C, D, z, nullptr, y, h, 1, 2, 32, 64, 64, F, nullptr), SSM_ERR_UNSUPPORTED,
           "ssd P != 64");
    if (ssm::g_launches != before) {
        std::printf("FAIL a rejected call launched work\n");
        ++failures;
    }

    // plans: host only
    ssm_fwd_plan_t pl{};
    expect(ssm_scan_fwd_plan(1, 2048, 131072, 16, H, nullptr, &pl), SSM_OK, "plan long context");
    if (pl.n_segments != 45 || pl.scratch_bytes != INT64_C(3) * 44 * 2048 * 16 * 4) {
        std::printf("FAIL long-context plan: %d segments, %lld bytes\n", pl.n_segments, (long long)pl.scratch_bytes);
        ++failures;
    }
    expect(ssm_scan_fwd_plan(8, 4096, 4096, 16, H, nullptr, &pl), SSM_OK, "plan 1.4B-like");
    if (pl.n_segments != 1 || pl.scratch_bytes != 0) {
        std::printf("FAIL 1.4B-like plan\n");
        ++failures;
    }
    ssm_fwd_opts_t po{};
    po.seg_len = 32;
    expect(ssm_scan_fwd_plan(1, 1, INT64_C(1) << 20, 16, F, &po, &pl), SSM_ERR_UNSUPPORTED, "plan too many segments");
    expect(ssm_scan_fwd_plan(1, 1, INT64_C(1) << 40, 16, F, nullptr, &pl), SSM_OK, "plan of a 2^40-step sequence");
    expect(ssm_scan_fwd_plan(1, 4, 16, 4, F, nullptr, nullptr), SSM_ERR_NULL, "plan null out");

    // calls that pass validation: a one-segment prefill reaches the launcher; a split one needs scratch,
    // which has no device here (SSM_ERR_HIP); the fixed-scratch variant needs none; decode and the fused
    // entry points reach their launchers
    const int l0 = ssm::g_launches;
    expect(ssm_scan_fwd(x, dl, A, B, C, D, z, y, h, 8, 4096, 64, 16, H, nullptr), SSM_OK, "one-segment prefill");
    expect(ssm_scan_fwd(x, dl, A, B, C, D, z, y, h, 1, 64, 8192, 16, H, nullptr), SSM_ERR_HIP, "split prefill, no device");
    expect(ssm_scan_fwd_noalloc(x, dl, A, B, C, D, z, y, h, 1, 64, 8192, 16, H, nullptr, nullptr), SSM_OK,
           "split prefill, fixed scratch");
    expect(ssm_scan_fwd_noalloc(x, dl, A, B, C, D, z, y, h, 1, 16384, 2048, 64, F, nullptr, &o), SSM_ERR_UNSUPPORTED,
           "noalloc with bad opts");
    o.lanes_per_channel = 0;
    o.seg_len = 32;
    expect(ssm_scan_fwd_noalloc(x, dl, A, B, C, D, z, y, h, 1, 16384, 2048, 64, F, nullptr, &o), SSM_ERR_SCRATCH,
           "noalloc beyond the fixed scratch");
    expect(ssm_scan_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, h, 2, 3, 0, 4, F, nullptr),
           SSM_OK, "L = 0 zeroes the state");
    expect(ssm_scan_step(h, x, dl, A, B, C, D, z, y, 512, 4096, 16, H, nullptr), SSM_OK, "decode step");
    expect(ssm_scan_step_conv(h, cs, x, A, D, 4, dl, D, 1, A, B, C, D, z, y, nullptr, 512, 4096, 16, H, nullptr), SSM_OK,
           "fused decode step");
    expect(ssm_scan_fwd_conv(x, A, D, cs, 4, dl, D, 1, A, B, C, D, z, nullptr, y, h, ffake(11), fake(12), 8, 4096, 4096,
                             16, H, nullptr),
           SSM_OK, "fused prefill");
    expect(ssm_conv1d_fwd(x, A, D, nullptr, y, h, 2, 4, 100, 4, 1, F, nullptr), SSM_OK, "conv1d");
    if (ssm::g_launches - l0 != 7) {
        std::printf("FAIL expected 7 launches, counted %d\n", ssm::g_launches - l0);
        ++failures;
    }
    for (int s = 0; s <= 7; ++s) std::printf("%s\n", ssm_status_string((ssm_status_t)s));
    if (failures) return 1;
    std::printf("abi driver: all host paths behaved\n");
    return 0;
}
