/*
 * dconv1d.h - C ABI of the MI355X (gfx950) pre-norm dilated Conv1d library.
 *
 * Two operations, both forward only, both enqueued asynchronously on a caller stream:
 *
 *   1. The pre-norm residual block
 *        out = x + Conv1d_{k=3, dilation=d, padding=d, stride=1, groups=1}(ReLU(BatchNorm1d_eval(x)))
 *      over (N, C, L) tensors, C -> C channels, so out has the shape of x.
 *      Source: POPCORNBENCH page "Kimi-K2.6__l2_p12" (pre-norm residual block problem),
 *      first turn: the block definition, the per-channel eval-mode BN formula with the
 *      running statistics, the conv's zero padding (taps t-d, t, t+d; out-of-range taps
 *      contribute nothing) and the output-length check that gives L_out = L.
 *      BN runs in eval mode (running statistics), in the *_train entry points in
 *      training mode (batch statistics and a running-statistics update), or, in the
 *      relu_dconv1d_residual_* entry points, outside the library (the caller passes the
 *      normalised activation and the residual separately).
 *
 *   2. Conv1d(k=3, stride 1) followed by GroupNorm.
 *      Source: POPCORNBENCH page "FW-GLM-5-1__l2_p35" (Conv1d + GroupNorm problem), its
 *      single turn: the conv index formula t_out*stride - padding + k*dilation, GroupNorm
 *      statistics per (sample, group) over the group's channels and all time steps with
 *      the biased variance, the optional affine gamma/beta, and the launcher's argument
 *      list (caller-allocated output, padding, dilation, num_groups, eps).
 *
 * Common rules for every compute entry point
 *   - Pointers marked "device" are device (HBM) addresses on the current HIP device
 *     (hipGetDevice); `stream` must belong to that device (0 = the null stream).
 *   - N == 0 (an empty batch) is valid: nothing is launched, x and out may be NULL.
 *   - Tensors are dense, row-major, no strides: x is [N][C][L] with L fastest, W is
 *     PyTorch's Conv1d layout [C_out][C_in][3].
 *   - Ownership: the caller owns and allocates every argument buffer, including out.
 *     The library owns a per-device workspace (folded BN scale/shift, repacked weights,
 *     GroupNorm partial statistics). It is allocated with hipMalloc on the first call
 *     that needs more than the current size (hipFree of the old one synchronises the
 *     device), kept for later calls, and freed by dconv1d_release().
 *   - All calls on one device share that workspace, and the library orders them: a
 *     call whose stream differs from that of the workspace's previous user makes its
 *     stream wait (on the device, through an event; the host does not block) for that
 *     call's kernels. Calls queued under stream capture skip this ordering (an event
 *     may not be waited on across the capture boundary); a captured call and calls on
 *     other streams must then be ordered by the caller. The single-launch GroupNorm
 *     path uses no workspace and needs no ordering.
 *   - No host synchronisation and no device-to-host reads happen on a call once the
 *     workspace is large enough; the call returns as soon as its kernels are queued.
 *   - Argument validation happens on the host before any HIP call; a rejected call
 *     touches no device state.
 *   - Return value: DCONV1D_OK (0) or a negative DCONV1D_E* code. dconv1d_last_error()
 *     then returns a message for the calling thread. Nothing aborts or throws across
 *     the ABI.
 */
#ifndef DCONV1D_H
#define DCONV1D_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DCONV1D_OK 0
/* A required pointer is NULL, a size is out of range (N < 0; a channel count below 1 or
 * above 16384; L outside [1, 2^30) for the block, T or padding outside [1, 2^29) /
 * [0, 2^29) for Conv1d + GroupNorm; d < 1; C_out % num_groups != 0; T_out < 1; eps < 0,
 * infinite or NaN), or an index would not fit the library's 32-bit per-sample indexing
 * (C*L >= 2^31). */
#define DCONV1D_EINVAL -1
/* `out` overlaps `x`. The kernels read x taps belonging to neighbouring output tiles
 * while other tiles are already writing out, so in-place operation is not supported. */
#define DCONV1D_EALIAS -2
/* A HIP runtime call or kernel launch failed (the message names the HIP error). */
#define DCONV1D_EHIP -3
/* The workspace could not be allocated. */
#define DCONV1D_ENOMEM -4

/*
 * prenorm_dconv1d_fwd - the pre-norm residual block in float32.
 *
 *   x            device, float32 [N][C][L]          input, also the residual
 *   running_mean device, float32 [C]                BN running mean
 *   running_var  device, float32 [C]                BN running variance
 *   gamma, beta  device, float32 [C]                BN affine weight and bias
 *   eps          BN epsilon, added to the variance inside the square root
 *   W            device, float32 [C][C][3]          conv weight, PyTorch layout
 *   b            device, float32 [C] or NULL        conv bias (NULL means zero)
 *   out          device, float32 [N][C][L]          result; must not overlap x
 *   N, C, L      batch, channels, length (N == 0 is a no-op that returns DCONV1D_OK)
 *   d            dilation; padding is d and the kernel size is 3 (any d >= 1; d >= L
 *                leaves only the centre tap)
 *   stream       HIP stream the work is queued on
 *
 * BN is the eval-mode form: scale = gamma/sqrt(var+eps), shift = beta - mean*scale,
 * folded once per call in double precision and rounded to float. The conv input is
 * zero-padded after the ReLU, so padded taps contribute exactly 0. Arithmetic:
 * float32 products, float32 accumulation (MFMA), bias and residual added in float32.
 * For most dilations the conv runs as Winograd F(2,3) over pairs of outputs d apart:
 * the same sum up to float32 rounding, with 2/3 of the multiply-adds
 * (dconv1d_block_method tells which form a shape takes).
 * The float32 entry points below that compute this block (training mode,
 * caller-normalised, no-allocation) choose the same way.
 */
int prenorm_dconv1d_fwd(const float* x, const float* running_mean, const float* running_var,
                        const float* gamma, const float* beta, float eps,
                        const float* W, const float* b, float* out,
                        int64_t N, int64_t C, int64_t L, int64_t d, hipStream_t stream);

/*
 * prenorm_dconv1d_fwd_noalloc - prenorm_dconv1d_fwd that allocates nothing, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Arguments, layout, arithmetic and results are those of prenorm_dconv1d_fwd (the same
 * kernels run). Limit: C <= 512 (DCONV1D_NOALLOC_MAX_C); larger C gives DCONV1D_EINVAL
 * with nothing queued. Instead of the workspace, the folded BN vectors and the
 * repacked weights go to a fixed device array inside the library (3 MiB + 4 KiB per
 * device, held until the process ends). No call allocates or frees device memory; the
 * first call on a device looks up that device's copy of the array once. Every call on
 * a device shares its array and overwrites what the previous call left there (nothing
 * in it needs clearing: each call writes all of it it reads). Calls that may overlap
 * in time on one device (different streams, or a replayed graph beside another call)
 * race on the array and give wrong results: the caller must order them. Calls of the
 * other entry points do not touch the array.
 */
#define DCONV1D_NOALLOC_MAX_C 512
int prenorm_dconv1d_fwd_noalloc(const float* x, const float* running_mean,
                                const float* running_var, const float* gamma,
                                const float* beta, float eps, const float* W, const float* b,
                                float* out, int64_t N, int64_t C, int64_t L, int64_t d,
                                hipStream_t stream);

/*
 * prenorm_dconv1d_fwd_bf16 - the same block with bfloat16 storage of x and out.
 *
 * x and out are bfloat16 bit patterns (uint16_t, [N][C][L]); every other argument is
 * as in prenorm_dconv1d_fwd (float32 parameters, W in float32 PyTorch layout). BN and
 * ReLU run in float32 on the bfloat16 x; the activation and W are rounded to bfloat16
 * (round to nearest even) for the bf16 MFMA, products accumulate in float32, bias and
 * the bfloat16 residual are added in float32, and out is rounded to bfloat16 (RNE).
 */
int prenorm_dconv1d_fwd_bf16(const uint16_t* x, const float* running_mean,
                             const float* running_var, const float* gamma, const float* beta,
                             float eps, const float* W, const float* b, uint16_t* out,
                             int64_t N, int64_t C, int64_t L, int64_t d, hipStream_t stream);

/*
 * prenorm_dconv1d_fwd_train - the pre-norm block with BatchNorm1d in training mode.
 *
 * Source: POPCORNBENCH page "Kimi-K2.6__l2_p97", first turn (training-mode BatchNorm:
 * normalise with the batch mean and the biased batch variance; the running mean and
 * variance move towards the batch mean and the n/(n-1)-corrected batch variance with
 * weight momentum), and "Kimi-K2.6__l2_p12", correctness-debugging turn (the block
 * with batch statistics taken per channel over the batch and time axes).
 *
 *   x, gamma, beta, eps, W, b, out, N, C, L, d, stream   as in prenorm_dconv1d_fwd
 *   running_mean device, float32 [C] or NULL   in/out: when given (with running_var),
 *   running_var  device, float32 [C] or NULL   updated in place with n = N*L:
 *                  running_mean = (1-momentum)*running_mean + momentum*mean
 *                  running_var  = (1-momentum)*running_var  + momentum*var*n/(n-1)
 *                Both NULL: no running update. Only one NULL: DCONV1D_EINVAL.
 *   momentum     weight of the batch statistics in the running update (finite)
 *   save_mean    device, float32 [C] or NULL   out: the batch mean
 *   save_invstd  device, float32 [C] or NULL   out: 1/sqrt(var + eps), biased var
 *
 * The batch statistics are mean and biased variance per channel over all N*L values;
 * N*L must be at least 2 (DCONV1D_EINVAL otherwise; N == 0 is a no-op that leaves
 * the running statistics unchanged). They are computed by a separate pass over x in
 * double precision with a fixed reduction order, so results are bitwise reproducible,
 * and folded into the same scale/shift as the eval-mode call; the conv is then the
 * eval-mode kernel. The running statistics and the saved vectors must not overlap x,
 * out or each other (DCONV1D_EALIAS).
 */
int prenorm_dconv1d_fwd_train(const float* x, float* running_mean, float* running_var,
                              const float* gamma, const float* beta, float eps, float momentum,
                              const float* W, const float* b, float* out,
                              float* save_mean, float* save_invstd,
                              int64_t N, int64_t C, int64_t L, int64_t d, hipStream_t stream);

/*
 * prenorm_dconv1d_fwd_train_bf16 - the training-mode block with bfloat16 storage of x and
 * out (uint16_t bit patterns); statistics are taken on the bfloat16 values of x, and the
 * rest is as in prenorm_dconv1d_fwd_train and prenorm_dconv1d_fwd_bf16.
 */
int prenorm_dconv1d_fwd_train_bf16(const uint16_t* x, float* running_mean, float* running_var,
                                   const float* gamma, const float* beta, float eps,
                                   float momentum, const float* W, const float* b, uint16_t* out,
                                   float* save_mean, float* save_invstd,
                                   int64_t N, int64_t C, int64_t L, int64_t d,
                                   hipStream_t stream);

/*
 * relu_dconv1d_residual_fwd - the block with the normalisation done by the caller:
 *        out = residual + Conv1d_{k=3, dilation=d, padding=d}(ReLU(xn))
 *
 * Source: POPCORNBENCH page "Kimi-K2.6__l2_p12", correctness-debugging turn: the
 * fallback that leaves BatchNorm to the framework (so it follows the module's train or
 * eval mode and keeps its running statistics) and fuses ReLU, the conv and the residual
 * add of the block input, which is passed separately from the normalised activation.
 *
 *   xn        device, float32 [N][C][L]          normalised activation (the conv input
 *                                                before ReLU)
 *   W, b      as in prenorm_dconv1d_fwd
 *   residual  device, float32 [N][C][L]          added to the conv output (the block's x)
 *   out       device, float32 [N][C][L]          result; must not overlap xn. It may be
 *                                                residual itself (in-place residual add),
 *                                                but not partially overlap it
 *                                                (DCONV1D_EALIAS)
 *   N, C, L, d, stream                            as in prenorm_dconv1d_fwd
 *
 * The conv input is zero-padded after the ReLU (padded taps contribute exactly 0), and
 * the arithmetic is that of prenorm_dconv1d_fwd with the BN step removed.
 */
int relu_dconv1d_residual_fwd(const float* xn, const float* W, const float* b,
                              const float* residual, float* out,
                              int64_t N, int64_t C, int64_t L, int64_t d, hipStream_t stream);

/*
 * relu_dconv1d_residual_fwd_bf16 - the same with bfloat16 storage of xn, residual and out
 * (uint16_t bit patterns); W and b stay float32, the arithmetic is that of
 * prenorm_dconv1d_fwd_bf16 with the BN step removed.
 */
int relu_dconv1d_residual_fwd_bf16(const uint16_t* xn, const float* W, const float* b,
                                   const uint16_t* residual, uint16_t* out,
                                   int64_t N, int64_t C, int64_t L, int64_t d,
                                   hipStream_t stream);

/*
 * conv1d_groupnorm_fwd - GroupNorm(Conv1d_{k=3, stride 1}(x)) in float32.
 *
 *   x            device, float32 [N][C_in][T]
 *   W            device, float32 [C_out][C_in][3]      conv weight, PyTorch layout
 *   bias         device, float32 [C_out] or NULL       conv bias (NULL means none)
 *   gamma, beta  device, float32 [C_out] or NULL       GroupNorm affine parameters; NULL
 *                                                      gamma means 1, NULL beta means 0
 *   eps          added to the biased group variance inside the square root
 *   num_groups   G; groups are contiguous blocks of C_out/G channels
 *   out          device, float32 [N][C_out][T_out], T_out = T + 2*padding - 2*dilation;
 *                must not overlap x
 *   padding >= 0, dilation >= 1; T_out must be >= 1
 *
 * When every group lies inside 16 output channels (C_out/num_groups divides 16),
 * C_in and C_out are multiples of 16, T_out <= 1024, W is 8-byte aligned and the input
 * window 128*ceil(T_out/128) + 2*dilation is at most 1216 steps, one kernel does it all:
 * the conv result stays on chip, the group statistics are reduced per (sample, group)
 * in a fixed order and out is written once; no workspace is used. Otherwise the conv
 * stores its result into out while writing per-(sample, channel, time tile) partial
 * sums and centred sums of squares to the workspace, and a second kernel merges them
 * per (sample, group) in a fixed order in double precision and normalises out in
 * place. Either way results are bitwise reproducible from run to run.
 *
 * The conv of the two-kernel path is Winograd F(2,3) too (see below) when padding equals
 * dilation and the rule of dconv1d_block_method, applied to (N, C_out, T, dilation),
 * picks that form.
 *
 * On the single-kernel path, dilation 1, 2 or 4 with a per-wave input window
 * (128 + 2*dilation + s <= 136 steps, s = (4 - padding % 4) % 4 when x is 16-byte
 * aligned and T % 4 == 0, else 0) and W 16-byte aligned take the Winograd F(2,3) form
 * of the conv: outputs t and t + dilation share three of their four inputs, and the
 * pair costs four products per input channel instead of six. The environment variable
 * DCONV1D_WINOGRAD = "0" selects the three-tap form instead (dconv1d_groupnorm_method
 * tells which form a call takes). Both forms sum in float32 and are bitwise
 * reproducible; their results differ in the last bits.
 */
int conv1d_groupnorm_fwd(const float* x, const float* W, const float* bias,
                         const float* gamma, const float* beta, float eps,
                         int64_t num_groups, float* out,
                         int64_t N, int64_t C_in, int64_t C_out, int64_t T,
                         int64_t padding, int64_t dilation, hipStream_t stream);

/* Message describing the last failed call on this thread ("" if none). The pointer
 * stays valid until the next library call on the same thread. */
const char* dconv1d_last_error(void);

/* Frees the workspace of every device. Waits for the device first (hipFree does).
 * Safe to call at any time when no library call is in flight; later calls reallocate. */
void dconv1d_release(void);

/*
 * Kernel timing for measurement tools. While enabled, each compute call records a
 * pair of HIP events on its stream around its dominant kernel (the fused conv kernel).
 * dconv1d_timer_read waits for the last recorded event, returns the summed duration
 * in milliseconds and the number of timed launches through the out-pointers, and
 * clears the record. At most 4096 launches are recorded between reads; later ones
 * are not timed. Returns DCONV1D_OK or DCONV1D_EHIP.
 */
int dconv1d_timer_enable(int enable);
int dconv1d_timer_read(double* total_ms, int64_t* launches);

/*
 * Which form of the conv a float32 block call of this shape (N, C, L, d) takes (the bf16
 * entry points always run the direct three-tap kernel). By default
 * DCONV1D_METHOD_WINOGRAD when L < 2^28; 3*P*c_w <= 2*L*c_d with P = ceil(L / (2*e)) * e
 * output pairs and e = min(d, L), where c_w and c_d are the two kernels' channel-tile
 * costs (each kernel takes 64*mb channels per workgroup, mb = 4, 2 or 1, whichever
 * minimises the padded channels divided by the tile's relative rate: 1, 0.96, 0.93 for
 * the Winograd kernel, 1, 0.98, 0.95 for the direct one; c_w = c_d when C is a multiple
 * of 256), each side scaled, when its grid fills at least one round of workgroups (per CU
 * as many as the tile's registers allow, times 256 CUs), by ceil(rounds) / rounds; else
 * DCONV1D_METHOD_DIRECT. On grids of fewer than two workgroups per compute
 * unit both kernels halve their channel tile (down to 64), which keeps the Winograd form
 * the faster one there too. The environment variable DCONV1D_WINOGRAD, read at every call,
 * overrides this: "0" selects the direct form always, "1" the Winograd form for every
 * L < 2^28. Returns DCONV1D_EINVAL for N < 0, C outside [1, 16384], L < 1 or d < 1.
 * Host only: no HIP call. Each form gives a sample the same bits at any N; as the
 * automatic choice depends on N, a sample's result may differ in its last bits between
 * batch sizes on either side of it (both within float32 rounding of the exact sum).
 */
#define DCONV1D_METHOD_DIRECT 0
#define DCONV1D_METHOD_WINOGRAD 1
int dconv1d_block_method(int64_t N, int64_t C, int64_t L, int64_t d);

/*
 * Which form of the conv a conv1d_groupnorm_fwd call with these arguments takes:
 * DCONV1D_METHOD_WINOGRAD or DCONV1D_METHOD_DIRECT (the three-tap kernels), on the
 * single-kernel or the two-kernel path, by the rules given at conv1d_groupnorm_fwd, the
 * DCONV1D_WINOGRAD override included. x and W are not dereferenced: only their alignment
 * matters (NULL stands for buffers aligned like every device allocation). Returns
 * DCONV1D_EINVAL for sizes conv1d_groupnorm_fwd rejects (N < 0, channels outside
 * [1, 16384], num_groups not dividing C_out, T outside [1, 2^29), padding outside
 * [0, 2^29), dilation < 1, T_out < 1, C*T above 2^31 - 1). Host only: no HIP call.
 */
int dconv1d_groupnorm_method(const float* x, const float* W, int64_t num_groups, int64_t N,
                             int64_t C_in, int64_t C_out, int64_t T, int64_t padding,
                             int64_t dilation);

#ifdef __cplusplus
}
#endif

#endif /* DCONV1D_H */
