/*
 * ssm_scan.h — C ABI of the MI355X (gfx950) selective state-space scan library, libssmscan.so.
 *
 * The operation (sources: page "State Space Models（SSM）とMamba" §2.1–§2.2 and §4.2; page
 * "Mambaとは？Transformer以外の系列モデル", sections 状態空間モデルを一つの式から理解する,
 * Mambaの核心は入力依存のDelta、B、C, Selective Scanは選択機構そのものではない, Mamba blockの
 * architecture and training、prefill、decodeでは計算の姿が違う):
 *
 *   for every batch row b and channel d, with a diagonal continuous-time A[d][·] and per-token
 *   step Δ_t, input matrices B_t and C_t (shared by all channels of the batch row):
 *     Ā_t[n] = exp(Δ_t · A[d][n])                        zero-order hold
 *     B̄_t[n] = (exp(Δ_t · A[d][n]) − 1) / A[d][n] · B_t[n]   (Δ_t · B_t[n] at A = 0, the limit)
 *     h_t[n] = Ā_t[n] · h_{t−1}[n] + B̄_t[n] · x_t         the recurrence (h_{−1} = 0 in prefill)
 *     y_t    = Σ_n C_t[n] · h_t[n] + D[d] · x_t            readout with the updated state + skip
 *     y_t    ← y_t · z_t · σ(z_t)                           optional SiLU gate
 *
 * Prefill (ssm_scan_fwd) evaluates the whole sequence; decode (ssm_scan_step) advances a stored
 * state by one token. Both compute in fp32 with an fp32 state.
 *
 * Conventions shared by every entry point
 *   - Pointers to tensors are DEVICE pointers owned by the caller; the library never frees them.
 *     All tensors are dense, row-major, with no padding:
 *       x, delta, z, y : [b][d][L]        (decode: [b][d])
 *       A              : [d][N]  fp32
 *       B, C           : [b][L][N]        (decode: [b][N])
 *       D              : [d]     fp32
 *       states         : [b][d][N] fp32
 *     `dtype` is the storage type of x, delta, z, B, C and y (SSM_F32 = float, SSM_BF16 = bf16 bit
 *     patterns, rounded to nearest-even on output). A, D and states are always fp32.
 *   - delta is used as given (a positive step; no softplus or bias is applied here).
 *   - Arguments are validated on the host before any launch; a failed check returns a non-zero
 *     status and launches nothing. Work is enqueued on `stream` (0 = the null stream) and the call
 *     returns without synchronising. Asynchronous device faults surface at the caller's next
 *     synchronisation of that stream.
 *   - Calls are reentrant: the library keeps no per-call global state. Calls on different streams
 *     may run concurrently. Calls that need scratch (a prefill split into time segments, the
 *     gradient pass, ssm_lti_fwd, ssm_ssd_fwd except bf16 with N of 64 or 128 and b·H at least
 *     twice the device's compute units) take it stream-ordered on `stream` from a memory pool the
 *     library creates on the current device at its first such call, and return it there at the
 *     end of the call. That pool keeps freed scratch (its release threshold is at the maximum), so
 *     repeated calls reuse it; it lives until the process ends. The device's default pool is not
 *     touched. ssm_scan_fwd_noalloc takes no scratch from any pool (see there).
 *   - NaN and Inf inputs propagate; nothing is clamped.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 1
#define SSM_MAX_N 64

/* Exported symbols (the library is built with hidden visibility by default). */
#if defined(__GNUC__)
#define SSM_API __attribute__((visibility("default")))
#else
#define SSM_API
#endif
/* The *_MAX_ENUM members are not values: they give both enums a 32-bit range, so any int a C or FFI
 * caller passes is a representable value of the type (and is then rejected or named "unknown"). */
typedef enum { SSM_F32 = 0, SSM_BF16 = 1, SSM_DTYPE_MAX_ENUM = 0x7fffffff } ssm_dtype_t;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_NULL = 1,        /* a required pointer is NULL                                   */
    SSM_ERR_SHAPE = 2,       /* a size is out of range (b, d, N < 1; L < 0; overflow)         */
    SSM_ERR_UNSUPPORTED = 3, /* N > SSM_MAX_N, unknown dtype, or an option value not accepted */
    SSM_ERR_HIP = 4,         /* a HIP runtime call or a launch failed                          */
    SSM_ERR_ALIAS = 5,       /* an output overlaps an input or another output                 */
    SSM_ERR_SCRATCH = 6,     /* ssm_scan_fwd_noalloc: the plan needs more than its fixed scratch */
    SSM_STATUS_MAX_ENUM = 0x7fffffff
} ssm_status_t;

/*
 * Prefill: the selective scan over a whole sequence (the parallel "prefill" mode), h_{−1} = 0.
 *   x, delta   [b][d][L] dtype      required
 *   A          [d][N] fp32          required; any finite value, A = 0 takes the ZOH limit
 *   B, C       [b][L][N] dtype      required
 *   D          [d] fp32             optional (NULL = no skip term)
 *   z          [b][d][L] dtype      optional (NULL = no gate)
 *   y          [b][d][L] dtype      required output; must not overlap any input
 *   final_state[b][d][N] fp32       optional output h_{L−1} (NULL = not written)
 *   b, d, N >= 1; L >= 0; N <= SSM_MAX_N. With L = 0 the call writes zeros to final_state (with
 *   ssm_scan_fwd_ex's initial_state: a copy of it) and touches nothing else, so x, delta, A, B, C, y may
 *   then be NULL.
 *   Errors: SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_UNSUPPORTED, SSM_ERR_ALIAS (nothing launched);
 *   SSM_ERR_HIP when scratch allocation or a launch fails (work already enqueued may have run).
 */
SSM_API ssm_status_t ssm_scan_fwd(const void *x, const void *delta, const float *A, const void *B,
                          const void *C, const float *D, const void *z, void *y,
                          float *final_state, int64_t b, int64_t d, int64_t L, int64_t N,
                          ssm_dtype_t dtype, hipStream_t stream);

/*
 * Decode: one recurrent step per (b, d) on a state kept in HBM (the recurrent "decode" mode).
 *   state      [b][d][N] fp32       required, in/out: read as h_{t−1}, overwritten with h_t
 *   x, delta   [b][d] dtype         required
 *   A          [d][N] fp32          required
 *   B, C       [b][N] dtype         required
 *   D          [d] fp32             optional
 *   z          [b][d] dtype         optional
 *   y          [b][d] dtype         required output
 *   b, d, N >= 1; N <= SSM_MAX_N; b * d < 2^31 (SSM_ERR_SHAPE otherwise). The state is read and
 *   written in place (it may not overlap any other argument). Errors as for ssm_scan_fwd.
 */
SSM_API ssm_status_t ssm_scan_step(float *state, const void *x, const void *delta, const float *A,
                           const void *B, const void *C, const float *D, const void *z, void *y,
                           int64_t b, int64_t d, int64_t N, ssm_dtype_t dtype, hipStream_t stream);

/*
 * Gradients of the prefill scan (ssm_scan_fwd with an optional initial state) for an upstream
 * gradient dy on y and, optionally, d_final_state on the final state. The forward map is the one
 * ssm_scan_fwd computes (page "Mambaとは？Transformer以外の系列モデル", section 状態空間モデルを一つの
 * 式から理解する); its derivatives follow by the chain rule in reverse time, and the forward states are
 * recomputed rather than stored (same page, section hardware-awareとは memory trafficまで設計すること).
 *   inputs            as for ssm_scan_fwd (x, delta, A, B, C, D, z), initial_state [b][d][N] fp32
 *                     or NULL (zeros)
 *   dy                [b][d][L] dtype, required
 *   d_final_state     [b][d][N] fp32 or NULL (zeros)
 *   dx, ddelta        [b][d][L] dtype, required outputs
 *   dz                [b][d][L] dtype; required when z is given, ignored otherwise
 *   dA                [d][N] fp32, required (summed over b and t)
 *   dB, dC            [b][L][N] fp32, required (summed over d)
 *   dD                [d] fp32 or NULL (summed over b and t; defined also when D is NULL)
 *   d_initial_state   [b][d][N] fp32 or NULL
 * The sums dA, dB, dC, dD are accumulated with float atomics, so their last bits can differ from
 * run to run; everything else is deterministic. Scratch (checkpoints every max(4, 32/states_per_lane) steps
 * and the segment aggregates) is taken stream-ordered from `stream` and returned. Outputs may not
 * overlap inputs or each other. b, d, N >= 1, L >= 1, N <= SSM_MAX_N. Errors as for ssm_scan_fwd.
 */
SSM_API ssm_status_t ssm_scan_bwd(const void *x, const void *delta, const float *A, const void *B,
                                  const void *C, const float *D, const void *z,
                                  const float *initial_state, const void *dy, const float *d_final_state,
                                  void *dx, void *ddelta, float *dA, float *dB, float *dC, float *dD,
                                  void *dz, float *d_initial_state, int64_t b, int64_t d, int64_t L,
                                  int64_t N, ssm_dtype_t dtype, hipStream_t stream);

/*
 * The short causal depthwise Conv1D (+ SiLU) of the Mamba block's main branch, which produces the
 * scan's x (page "Mambaとは？Transformer以外の系列モデル", section Mamba blockのarchitecture), and its
 * decode step with the per-layer Conv1D state (same page, section training、prefill、decodeでは計算の
 * 姿が違う). Per channel d with taps w[d][0..W) and bias c_d:
 *     u_t = c_d + Σ_{k<W} w[d][k] · xin_{t−(W−1)+k},   x_t = silu(u_t) if apply_silu, else u_t,
 * the inputs before t = 0 taken from state_in (zeros when NULL).
 *   xin, x_out        [b][d][L] dtype (x_out may not overlap xin)
 *   w                 [d][W] fp32, 1 <= W <= SSM_MAX_CONV_W
 *   bias              [d] fp32 or NULL
 *   state_in          [b][d][W−1] fp32 or NULL: the W−1 inputs before the sequence, oldest first
 *   state_out         [b][d][W−1] fp32 or NULL: the last W−1 inputs after it (may equal state_in)
 * b, d >= 1, L >= 0. Errors as for ssm_scan_fwd.
 */
#define SSM_MAX_CONV_W 8
SSM_API ssm_status_t ssm_conv1d_fwd(const void *xin, const float *w, const float *bias, const float *state_in,
                                    void *x_out, float *state_out, int64_t b, int64_t d, int64_t L, int64_t W,
                                    int32_t apply_silu, ssm_dtype_t dtype, hipStream_t stream);

/* Decode: one new input per (b, d). state [b][d][W−1] fp32 is read and shifted in place (the new
 * input enters last); xin, x_out [b][d] dtype. Other arguments as for ssm_conv1d_fwd. */
SSM_API ssm_status_t ssm_conv1d_step(float *state, const void *xin, const float *w, const float *bias,
                                     void *x_out, int64_t b, int64_t d, int64_t W, int32_t apply_silu,
                                     ssm_dtype_t dtype, hipStream_t stream);

/*
 * The main branch of the Mamba block from the Conv1D's input to y in one pass: the Conv1D + SiLU of
 * ssm_conv1d_fwd (apply_silu on) and the scan of ssm_scan_fwd, with the parameter preprocessing folded
 * into the scan's tile staging (page "Mambaとは？Transformer以外の系列モデル", section hardware-awareとは
 * memory trafficまで設計すること: parameter generation, discretisation and scan in one kernel, only the
 * outputs going back to memory; section Mamba blockのarchitecture: Conv1D, SiLU, then the selective SSM).
 * Per (b, d) and t:
 *     x_t = silu(c_d + Σ_{k<W} conv_w[d][k] · xin_{t−(W−1)+k})        (inputs before t = 0 from
 *                                                                     conv_state_in, else zeros)
 *     Δ_t = softplus(delta_t + delta_bias[d]) if delta_softplus, else delta_t + delta_bias[d]
 * then the scan of ssm_scan_fwd on x, Δ from initial_state (zeros when NULL). The convolved x is kept in
 * fp32 inside the kernel (it is not rounded to the storage type before the scan); x_out, when given,
 * receives it rounded to the storage type (for the caller's projections of x).
 *   xin                [b][d][L] dtype, required
 *   conv_w             [d][W] fp32, required, 1 <= W <= SSM_MAX_FUSED_CONV_W (SSM_ERR_UNSUPPORTED above)
 *   conv_bias          [d] fp32 or NULL
 *   conv_state_in      [b][d][W−1] fp32 or NULL: the W−1 inputs before the sequence, oldest first
 *   delta              [b][d][L] dtype, required: Δ before its bias and softplus
 *   delta_bias         [d] fp32 or NULL
 *   A, B, C, D, z      as for ssm_scan_fwd; initial_state [b][d][N] fp32 or NULL
 *   y, final_state     as for ssm_scan_fwd
 *   conv_state_out     [b][d][W−1] fp32 or NULL: the last W−1 inputs after the sequence (must not
 *                      overlap conv_state_in; copy it back for the next call)
 *   x_out              [b][d][L] dtype or NULL
 * Scratch as for ssm_scan_fwd. No output may overlap an input or another output. Errors as for
 * ssm_scan_fwd.
 */
#define SSM_MAX_FUSED_CONV_W 4
SSM_API ssm_status_t ssm_scan_fwd_conv(const void *xin, const float *conv_w, const float *conv_bias,
                                       const float *conv_state_in, int64_t W, const void *delta,
                                       const float *delta_bias, int32_t delta_softplus, const float *A,
                                       const void *B, const void *C, const float *D, const void *z,
                                       const float *initial_state, void *y, float *final_state,
                                       float *conv_state_out, void *x_out, int64_t b, int64_t d, int64_t L,
                                       int64_t N, ssm_dtype_t dtype, hipStream_t stream);

/*
 * One decode step of the same branch in one launch (page "Mambaとは？Transformer以外の系列モデル", section
 * training、prefill、decodeでは計算の姿が違う: each layer keeps a Conv1D state and an SSM state): the token's
 * raw input is convolved with conv_state (the last W−1 inputs, fp32 [b][d][W−1], shifted in place; may be
 * NULL when W = 1), SiLU, Δ as in ssm_scan_fwd_conv, then the step of ssm_scan_step on state.
 *   state [b][d][N] fp32 in/out; xin, delta, z, y, x_out (nullable) [b][d] dtype; conv_w [d][W];
 *   conv_bias, delta_bias [d] or NULL; A, B, C, D as for ssm_scan_step.
 * The two states and the outputs may not overlap each other or any input. Errors as for ssm_scan_step.
 */
SSM_API ssm_status_t ssm_scan_step_conv(float *state, float *conv_state, const void *xin, const float *conv_w,
                                        const float *conv_bias, int64_t W, const void *delta,
                                        const float *delta_bias, int32_t delta_softplus, const float *A,
                                        const void *B, const void *C, const float *D, const void *z, void *y,
                                        void *x_out, int64_t b, int64_t d, int64_t N, ssm_dtype_t dtype,
                                        hipStream_t stream);

/*
 * The time-invariant (LTI) case evaluated as a convolution (page "State Space Models（SSM）とMamba" §2.3;
 * page "Mambaとは？Transformer以外の系列モデル", section 固定SSMには「再帰」と「畳み込み」の二つの顔がある):
 * when Ā, B̄ and C are the same at every step, the zero-state recurrence is y = x ∗ K̄ with
 * K̄ = (CB̄, CĀB̄, CĀ²B̄, …), which the FFT evaluates in O(L log L). Every channel is its own system.
 *
 * ssm_lti_kernel: K[d][k] = Σ_n C[d][n] · Ā^k · B̄ for k < L, with the ZOH of ssm_scan_fwd
 * (Ā = exp(delta[d]·A[d][n]), B̄ = (Ā − 1)/A · B[d][n], Δ·B at A = 0).
 *   delta [d], A, B, C [d][N], K [d][L] (output); all fp32. d, N >= 1, N <= SSM_MAX_N, 0 <= L < 2^24.
 *
 * ssm_lti_conv: y[b][d][t] = Σ_{s<=t} K[d][t−s] · x[b][d][s] + D[d] · x[b][d][t], times silu(z) when z
 * is given, by FFT (two batch rows of a channel per complex transform of 2^⌈log2 2L⌉ >= 1024 points).
 *   x, z, y [b][d][L] dtype (z may be NULL); K [d][L] fp32 (any kernel, e.g. from ssm_lti_kernel);
 *   D [d] fp32 or NULL. y may not overlap the inputs. b >= 1, 1 <= d <= 2^22,
 *   1 <= L <= SSM_LTI_MAX_L (SSM_ERR_UNSUPPORTED above it).
 *
 * ssm_lti_fwd: both: K̄ into scratch taken stream-ordered from `stream`, then the convolution; any L >= 1
 * (below 2^40). Up to SSM_LTI_MAX_L steps: K̄ over L taps (d·L·4 bytes of scratch) and one transform per
 * row pair. Longer: chunks of SSM_LTI_CHUNK steps, each convolved with K̄ over SSM_LTI_CHUNK taps, joined
 * through the state, the other face of the same system (same page and section): each chunk's end state
 * from zero, E_n = B̄_n·Σ_s Ā_n^{chunk−1−s}·x_s, is chained by h ← Ā^chunk·h + E into the state entering every
 * later chunk, whose response Σ_n C_n·Ā_n^{τ+1}·h_n that chunk adds to its output τ steps in (scratch:
 * d·SSM_LTI_CHUNK + b·d·(n_chunks − 1)·N floats). No final state is produced (the convolution form has none;
 * ssm_scan_fwd with the parameters repeated over t gives it). Errors as for ssm_scan_fwd.
 */
#define SSM_LTI_MAX_L 8192
#define SSM_LTI_CHUNK 4096
SSM_API ssm_status_t ssm_lti_kernel(const float *delta, const float *A, const float *B, const float *C, float *K,
                                    int64_t d, int64_t L, int64_t N, hipStream_t stream);
SSM_API ssm_status_t ssm_lti_conv(const void *x, const float *K, const float *D, const void *z, void *y, int64_t b,
                                  int64_t d, int64_t L, ssm_dtype_t dtype, hipStream_t stream);
SSM_API ssm_status_t ssm_lti_fwd(const void *x, const float *delta, const float *A, const float *B, const float *C,
                                 const float *D, const void *z, void *y, int64_t b, int64_t d, int64_t L, int64_t N,
                                 ssm_dtype_t dtype, hipStream_t stream);

/*
 * The scalar-decay selective SSM of Mamba-2's state space duality (page "State Space Models（SSM）とMamba"
 * §4.6 relates SSMs and linear attention; the pages give no formulas, so this is the selective scan of
 * ssm_scan_fwd with A restricted to one scalar per head). Channels come in H heads of P; head h has the
 * decay a_h (A[d][n] = a_h for its channels and all states) and one step delta[b][h][t] shared by its P
 * channels. Unrolled, y = (causal mask ∘ e^{a(c_t − c_s)} ∘ C Bᵀ)(β ∘ x) + D x per head, a masked linear
 * attention; it is evaluated chunk by chunk (64 steps) with matrix products on the MFMA units (fp32
 * products for fp32 storage; bf16 products, fp32 operands entering as bf16 hi + lo, for bf16 storage).
 *   x, z, y           [b][H·P][L] dtype (z may be NULL)
 *   delta             [b][H][L] dtype
 *   A                 [H] fp32 (the per-head decay a_h)
 *   B, C              [b][L][N] dtype (shared by all heads)
 *   D                 [H·P] fp32 or NULL
 *   initial_state     [b][H·P][N] fp32 or NULL (zeros); final_state [b][H·P][N] fp32 or NULL
 * Supported: P = 64, N in {32, 64, 128} (SSM_ERR_UNSUPPORTED otherwise); b, H >= 1, L >= 0. Scratch of
 * b·H·⌈L/64⌉·(P·N + 1) floats is taken stream-ordered from `stream`, except for bf16 storage with N of 64
 * or 128 and b·H at least twice the device's compute units, which needs none (the whole form then runs
 * as one ordered walk per (b, head)). Errors as for ssm_scan_fwd.
 */
SSM_API ssm_status_t ssm_ssd_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C,
                                 const float *D, const void *z, const float *initial_state, void *y,
                                 float *final_state, int64_t b, int64_t H, int64_t P, int64_t L, int64_t N,
                                 ssm_dtype_t dtype, hipStream_t stream);

/*
 * Options of ssm_scan_fwd_ex. Zero-initialise, then set what you need; zero means "choose".
 *   seg_len            time-segment length (multiple of 32) carried across by the chunk-carry
 *                      pass; 0 = chosen from the shape, >= L = one segment
 *   lanes_per_channel  1, 2 or 4 lanes of a wavefront share one channel's N states (a wavefront
 *                      then covers 64 / this channels; each lane holds at most 16 states);
 *                      0 = chosen from the shape
 *   initial_state    [b][d][N] fp32 device pointer, h_{−1} (NULL = zeros); lets a caller
 *                    continue a sequence that an earlier call ended (pass its final_state)
 *   ev_begin, ev_end hipEvent_t values (may be NULL); when set, the dispatch of the output-pass
 *                    kernel of the fast (scaled-state) path sets them at its start and end, for
 *                    timing that kernel alone (hipExtLaunchKernel's start/stop events)
 */
typedef struct {
    int32_t seg_len;
    int32_t lanes_per_channel;
    const float *initial_state;
    void *ev_begin;
    void *ev_end;
    int64_t reserved[4];
} ssm_fwd_opts_t;

/* ssm_scan_fwd with explicit options (opts may be NULL = all defaults). */
SSM_API ssm_status_t ssm_scan_fwd_ex(const void *x, const void *delta, const float *A, const void *B,
                             const void *C, const float *D, const void *z, void *y,
                             float *final_state, int64_t b, int64_t d, int64_t L, int64_t N,
                             ssm_dtype_t dtype, hipStream_t stream, const ssm_fwd_opts_t *opts);

/* The launch plan ssm_scan_fwd_ex would use for this shape and these options (host only, no
 * device work), planned for a 256-CU device (MI355X): the resolved segment length, lanes per
 * channel and states per lane, the number of segments, the one-wavefront workgroups of each
 * segment and of each pass, and the scratch bytes. Returns SSM_OK or the validation error. */
typedef struct {
    int32_t seg_len;
    int32_t lanes_per_channel;
    int32_t states_per_lane;
    int32_t n_segments;
    int64_t waves_per_segment;
    int64_t groups_output_pass;
    int64_t groups_aggregate_pass;
    int64_t scratch_bytes;
} ssm_fwd_plan_t;

SSM_API ssm_status_t ssm_scan_fwd_plan(int64_t b, int64_t d, int64_t L, int64_t N, ssm_dtype_t dtype,
                               const ssm_fwd_opts_t *opts, ssm_fwd_plan_t *plan);

/*
 * ssm_scan_fwd_ex that allocates nothing, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, and harnesses that forbid allocation. Same arguments, plan,
 * kernels and results as ssm_scan_fwd_ex. The scratch of a time-split plan (the segment aggregates,
 * and the carries past 16 segments: ssm_fwd_plan_t.scratch_bytes) lives in a fixed device array of
 * SSM_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds from its first use until the
 * process ends; no hipMalloc, hipFree or allocating library routine is called. A plan needing more
 * returns SSM_ERR_SCRATCH and launches nothing (a longer seg_len in opts shrinks it). Every call on a
 * GPU shares that GPU's array, which keeps the last call's contents: calls that overlap on one GPU
 * (different streams, or host threads) race and must be serialised by the caller. Nothing in the
 * array needs clearing: a call writes every scratch word before reading it. Other errors as for
 * ssm_scan_fwd.
 */
#define SSM_NOALLOC_SCRATCH_BYTES (32ll << 20)
SSM_API ssm_status_t ssm_scan_fwd_noalloc(const void *x, const void *delta, const float *A, const void *B,
                                          const void *C, const float *D, const void *z, void *y,
                                          float *final_state, int64_t b, int64_t d, int64_t L, int64_t N,
                                          ssm_dtype_t dtype, hipStream_t stream, const ssm_fwd_opts_t *opts);

/* Human-readable name of a status code (static string, never NULL). */
SSM_API const char *ssm_status_string(ssm_status_t s);

/* SSM_ABI_VERSION of the loaded library. */
SSM_API int ssm_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SSM_SCAN_H */
