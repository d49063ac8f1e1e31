// launch.h — private host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_scan.h"

namespace ssm {

// Everything the prefill launchers need; validated by the ABI layer beforehand.
struct FwdLaunch {
    const void *x, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z;
    void *y;
    float *final_state;
    const float *init_state;  // h_{-1} of segment 0, or nullptr (zeros)
    int64_t b, d, L, N;
    bool bf16;
    int lanes_per_channel;    // G = 1, 2 or 4 lanes share one channel (64 / G channels per wavefront)
    int states_per_lane;      // 4, 8 or 16, with lanes_per_channel * states_per_lane >= N
    int64_t seg_len;          // multiple of kSegQuantum
    int n_seg;                // ceil(L / seg_len) >= 1
    float *scratch;           // scratch_floats(n_seg, b, d, N) floats
    hipEvent_t ev_begin, ev_end;
    float *ckpt;              // optional: states entering every ck_len-th step, [b][d][ceil(L/ck_len)][N]
    int ck_len;               // checkpoint interval (ckpt_len) when ckpt is set
    // fused front end (set conv_w to enable; then x is the Conv1D's raw input): Conv1D (conv_W <= 4 taps,
    // bias) + SiLU gives the scan's x; Δ = delta + delta_bias, through softplus when delta_softplus
    const float *conv_w, *conv_bias, *conv_state_in, *delta_bias;
    float *conv_state_out;
    void *x_out;
    int conv_W, delta_softplus;
    // the small-problem kernel (small_problem() holds and no option forced a plan): no scratch, no segments
    bool small;
};

// Small problems: at most kSmallMaxBlocks blocks of 16 channels over 2·kSmallSeg < L <= kSmallSeg·kSmallMaxWaves
// steps with N <= 16 run as one workgroup per block, one wavefront per kSmallSeg steps (scan_small.hip).
constexpr int kSmallSeg = 16;
constexpr int kSmallMaxWaves = 16;
constexpr int kSmallCh = 16;  // channels per workgroup
constexpr int64_t kSmallMaxBlocks = 256;
inline bool small_problem(int64_t b, int64_t d, int64_t L, int64_t N) {
    return N <= 16 && L > 2 * kSmallSeg && L <= (int64_t)kSmallSeg * kSmallMaxWaves &&
           b * ((d + kSmallCh - 1) / kSmallCh) <= kSmallMaxBlocks;
}
// Steps per wavefront: half of kSmallSeg where kSmallMaxWaves such segments cover the sequence.
inline int small_seg(int64_t L) {
    return L <= (int64_t)(kSmallSeg / 2) * kSmallMaxWaves ? kSmallSeg / 2 : kSmallSeg;
}
hipError_t launch_scan_small(const FwdLaunch &p, hipStream_t stream);

// Everything the gradient launcher needs (validated by the ABI layer).
struct BwdLaunch {
    const void *x, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z;
    const float *init_state;     // nullable
    const void *dy;
    const float *d_final_state;  // nullable
    void *dx, *ddelta, *dz;      // dz nullable (required when z is given)
    float *dA, *dB, *dC, *dD;    // dD nullable
    float *d_init_state;         // nullable
    int64_t b, d, L, N;
    bool bf16;
    int lanes_per_channel, states_per_lane;
    int64_t seg_len;             // time split of the checkpointing forward pass
    int n_seg;
    int64_t grad_seg_len;        // time split of the reverse aggregate and gradient passes
    int grad_n_seg;
    float *scratch;              // bwd_scratch_floats(...) floats
};

hipError_t launch_scan_bwd(const BwdLaunch &p, hipStream_t stream);

// Aggregate pass of a time split (agg_rev.hip): for segments 0 .. n_seg − 2, P = Π Ā = exp(A·ΣΔ) and E, the
// end state from zero, both [n_seg − 1][b][d][N] fp32, by a backward walk that stops once the decay back
// to the step reached is at most 2^-24 for every state of a wavefront. N <= 64.
struct AggLaunch {
    const void *x, *delta;
    const float *A;
    const void *B;
    float *P, *E;
    // E2 (may be null): when given, the walk of state group 0 (states 0..3) is split between two wavefronts
    // per unit, and the earlier part's sum goes to E2 [n_seg-1][b][d][N] (states 0..3 only), to be added
    // to E by the carry pass; E then holds the later part's
    float *E2;
    int64_t b, d, L, N, seg_len;
    int n_seg;
    bool bf16;
};
hipError_t launch_agg_rev(const AggLaunch &p, hipStream_t stream);

// Causal depthwise Conv1D (+ SiLU) over [b][d][L] rows, and its decode step.
struct ConvLaunch {
    const void *xin;
    const float *w, *bias, *state_in;  // bias, state_in nullable
    void *xout;
    float *state_out;                  // nullable; may equal state_in
    int64_t b, d, L;
    int W;                             // 1 .. 8 taps
    int silu_on;
    bool bf16;
};
struct ConvStepLaunch {
    float *state;                      // [b][d][W-1], updated in place
    const void *xin;                   // [b][d]
    const float *w, *bias;
    void *xout;                        // [b][d]
    int64_t b, d;
    int W, silu_on;
    bool bf16;
};
hipError_t launch_conv1d(const ConvLaunch &p, hipStream_t stream);

// LTI convolution form: the kernel K̄ and its FFT convolution with x (transform sizes 2^10 … 2^14).
constexpr int kLtiMinLog2 = 10;
constexpr int kLtiMaxLog2 = 14;
struct LtiKernelLaunch {
    const float *delta, *A, *B, *C;
    float *K;
    int64_t d, L, N;
};
struct LtiConvLaunch {
    const void *x, *z;                 // z nullable
    const float *K, *D;                // D nullable
    void *y;
    int64_t b, d, L;
    bool bf16;
    // Chunked form (chunk > 0): K holds `chunk` taps per channel, every chunk of the sequence is convolved
    // on its own, and each chunk after the first adds the response Σ_n C_n·Ā_n^{τ+1}·h_n of the state h
    // entering it: h_in [b][d][n_chunks − 1][N]; delta [d], A, C [d][N] give Ā and C.
    int64_t chunk;
    const float *h_in, *delta, *A, *C;
    int64_t N;
};
int lti_fft_log2(int64_t L);           // log2 of the transform size used for sequence length L
hipError_t launch_lti_kernel(const LtiKernelLaunch &p, hipStream_t stream);
hipError_t launch_lti_conv(const LtiConvLaunch &p, hipStream_t stream);

// Chunk length of the chunked LTI form (sequences longer than one transform), and the states it passes:
// H [b][d][n_chunks − 1][N] = the state at the end of chunks 0 .. n_chunks − 2 (from zero at t = 0).
constexpr int64_t kLtiChunk = SSM_LTI_CHUNK;
struct LtiChunkLaunch {
    const void *x;
    const float *delta, *A, *B;
    float *H;
    int64_t b, d, L, N, chunk;
    bool bf16;
};
hipError_t launch_lti_chunk_states(const LtiChunkLaunch &p, hipStream_t stream);

// Scalar-decay (state space duality) form, chunked on the MFMA units: heads of 64 channels, N in {32, 64, 128}.
struct SsdLaunch {
    const void *x, *delta, *B, *C, *z;   // z nullable
    const float *A, *D, *h0;             // D, h0 nullable
    void *y;
    float *hT;                           // nullable
    float *scratch;                      // ssd_scratch_floats(b, H, L, N, bf16, cus) floats, or null
    int64_t b, H, L, N;
    bool bf16;
    int cus;                             // compute units of the device
};
// The single walk (ssd_fused_kernel) serves bf16 storage with N of 64 or 128 once b·H gives every CU two
// workgroups; it needs no scratch. The other forms take ssd_scratch_floats(...) floats.
bool ssd_single_walk(int64_t b, int64_t H, int64_t N, bool bf16, int cus);
int64_t ssd_scratch_floats(int64_t b, int64_t H, int64_t L, int64_t N, bool bf16, int cus);
hipError_t launch_ssd(const SsdLaunch &p, hipStream_t stream);
hipError_t launch_conv_step(const ConvStepLaunch &p, hipStream_t stream);

struct StepLaunch {
    float *state;
    const void *x, *delta;
    const float *A;
    const void *B, *C;
    const float *D;
    const void *z;
    void *y;
    int64_t b, d, N;
    bool bf16;
    // fused front end (conv_w set: x is the Conv1D's raw input, conv_state [b][d][conv_W − 1] is shifted in
    // place, x_out (nullable) receives the convolved input); as in FwdLaunch
    float *conv_state;
    const float *conv_w, *conv_bias, *delta_bias;
    void *x_out;
    int conv_W, delta_softplus;
};

hipError_t launch_scan_fwd(const FwdLaunch &p, hipStream_t stream);
hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t stream);
hipError_t launch_scan_step(const StepLaunch &p, hipStream_t stream);

// Fixed scratch of ssm_scan_fwd_noalloc (SSM_NOALLOC_SCRATCH_BYTES in the public header): its address on
// the current device, looked up once per device.
constexpr int64_t kNoAllocScratchBytes = INT64_C(32) << 20;
hipError_t noalloc_scratch(float **out);

constexpr int kSegQuantum = 32; // time segments are multiples of this many steps
constexpr int64_t kAggWalkMinSeg = 1024;  // segments this long take the truncated backward aggregate walk
constexpr int kFoldMaxSeg = 16; // up to this many segments the output pass chains the carry itself

// Scratch floats of a time-split prefill: aggregates P and E, plus the carries when a separate
// carry kernel chains them.
inline int64_t scratch_floats(int64_t n_seg, int64_t b, int64_t d, int64_t N) {
    if (n_seg <= 1) return 0;
    return (n_seg > kFoldMaxSeg ? 3 : 2) * (n_seg - 1) * b * d * N;
}

// Gradient pass: checkpoint interval (steps whose states fit one lane's registers) and scratch:
// the forward pass's scratch, the checkpoints, and the reverse aggregates (Π Ā, adjoint from zero).
inline int ckpt_len(int states_per_lane) { return (32 / states_per_lane) < 4 ? 4 : 32 / states_per_lane; }
inline int64_t bwd_scratch_floats(int64_t n_seg, int64_t grad_n_seg, int64_t b, int64_t d, int64_t L, int64_t N,
                                  int npl) {
    const int64_t ck = ckpt_len(npl);
    return scratch_floats(n_seg, b, d, N) + b * d * ((L + ck - 1) / ck) * N + 2 * (grad_n_seg - 1) * b * d * N;
}

}  // namespace ssm
