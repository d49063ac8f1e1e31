// stubs.cpp — stand-ins for the kernel launchers of libssmscan.so, so that the host code of abi.cpp
// (validation, planning, scratch handling, dispatch) can be built with the address and undefined-behaviour
// sanitizers and run on a machine without a GPU. Every launcher counts its call and returns success; none
// touches device memory.
#include "launch.h"

namespace ssm {

int g_launches = 0;

hipError_t launch_scan_fwd(const FwdLaunch &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fill_zero(float *, int64_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_scan_small(const FwdLaunch &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_scan_step(const StepLaunch &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_scan_bwd(const BwdLaunch &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_conv1d(const ConvLaunch &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_conv_step(const ConvStepLaunch &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_lti_kernel(const LtiKernelLaunch &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_lti_conv(const LtiConvLaunch &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_lti_chunk_states(const LtiChunkLaunch &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_ssd(const SsdLaunch &, hipStream_t) { ++g_launches; return hipSuccess; }

int lti_fft_log2(int64_t L) {
    int m = kLtiMinLog2;
    while ((int64_t(1) << m) < 2 * L) ++m;
    return m;
}
bool ssd_single_walk(int64_t, int64_t, int64_t, bool, int) { return false; }
int64_t ssd_scratch_floats(int64_t b, int64_t H, int64_t L, int64_t N, bool, int) {
    return b * H * ((L + 63) / 64) * (64 * N + 1);
}
hipError_t noalloc_scratch(float **out) {
    static float stand_in[16];
    *out = stand_in;
    return hipSuccess;
}

}  // namespace ssm
