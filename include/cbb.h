/*
 * cbb.h -- C ABI of libcbb.so, the backward pass of a Darknet/Caffe-style
 * convolutional block on an AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title, address):
 *  [P1] "YOLOv3 backpropagation: full-flow source analysis"
 *       (suzhouguqin.com/content/1291550.html)
 *  [P2] "Caffe source study ch.4 (5): the LeNet backward pass"
 *       (csdndocs.com/article/9344743)
 *  [P3] "AlexeyAB DarkNet analysis (4): network forward/backward and the layer struct"
 *       (m.dandelioncloud.cn/article/details/1675816420510003202)
 *  [P4] "caffe source study -- one article is enough"
 *       (geek-share.com/detail/2722348220.html)
 *  [P5] "Understanding BatchNorm" (javaforall.cn/143067.html)
 *
 * Conventions shared by every entry point
 *  - Tensor pointers are DEVICE pointers owned by the caller; fp32 unless
 *    noted; activations NCHW-contiguous (the delta/output layout of the layer
 *    struct in [P3]); conv weights OIHW; inner-product weights out x in.
 *  - Nothing here allocates device memory or synchronises the host.  Every
 *    call validates its arguments on the host (before touching the GPU),
 *    enqueues its kernels on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream) and returns.  Scratch memory comes from a
 *    caller-provided `workspace` whose size the matching *_workspace_size
 *    call reports.
 *  - Parameter gradients (dw, db, dgamma, dbeta) ACCUMULATE (+=), as the
 *    beta = 1 gemm/gemv calls of [P1] section 3.1 and [P2] layers 4 and 8
 *    do, so a caller sums several batches by calling again; zero them first
 *    for a single batch.
 *  - Input gradients are skipped when their pointer is NULL (the NULL
 *    net.delta of the first layer, [P3] backward_network); otherwise they are
 *    overwritten, or added onto when `*_accumulate` is 1 (an input feeding
 *    several consumers receives the sum of their gradients).
 *  - Results are deterministic: no floating-point atomics; repeated calls on
 *    the same inputs give bitwise identical outputs.
 *  - Errors are returned as a negative cbb_status and nothing is enqueued;
 *    the pages abort instead (assert / CHECK).
 */
#ifndef CBB_H
#define CBB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CBB_ABI_VERSION 2

typedef enum cbb_status {
  CBB_OK = 0,
  CBB_EINVAL = -1,        /* NULL required pointer, non-positive size, bad enum value */
  CBB_ESHAPE = -2,        /* geometry yields an empty or inconsistent output          */
  CBB_EUNSUPPORTED = -3,  /* valid but not implemented (e.g. ksize > 7, scale > 8)     */
  CBB_EWORKSPACE = -4,    /* workspace NULL or smaller than the reported size         */
  CBB_EHIP = -5,          /* a HIP launch failed; cbb_last_error() has its text       */
  CBB_ESCRATCH = -6       /* needs more scratch than CBB_NOALLOC_SCRATCH_BYTES        */
} cbb_status;

/* Activation whose gradient is taken, read from the activation OUTPUT y as
 * Darknet's *_gradient functions do ([P1] section 7):
 *   LINEAR 1;  LEAKY (y > 0) ? 1 : slope;  LOGISTIC (1 - y) y;  RELU (y > 0);
 *   TANH 1 - y^2;  ELU (y >= 0) ? 1 : y + 1;  SELU (y >= 0) ? 1.0507 : y + 1.0507 * 1.6732;
 *   PLSE (y < 0 || y > 1) ? .01 : .125;  LHTAN (0 < y < 1) ? 1 : .001;
 *   HARDTAN (-1 < y < 1) ? 1 : 0;  STAIR (floor(y) == y) ? 0 : 1;  RAMP (y > 0) + .1;
 *   RELIE (y > 0) ? 1 : .01;  LOGGY 2 (1 - s) s with s = (y + 1) / 2.
 * The networks on the pages use the first four; the slope applies to LEAKY only. */
typedef enum cbb_act {
  CBB_ACT_LINEAR = 0,
  CBB_ACT_LEAKY = 1,
  CBB_ACT_LOGISTIC = 2,
  CBB_ACT_RELU = 3,
  CBB_ACT_TANH = 4,
  CBB_ACT_ELU = 5,
  CBB_ACT_SELU = 6,
  CBB_ACT_PLSE = 7,
  CBB_ACT_LHTAN = 8,
  CBB_ACT_HARDTAN = 9,
  CBB_ACT_STAIR = 10,
  CBB_ACT_RAMP = 11,
  CBB_ACT_RELIE = 12,
  CBB_ACT_LOGGY = 13
} cbb_act;

/* Batch-norm mode of a block (cbb_conv_desc.batch_normalize):
 *   NONE  no BN; the conv has a bias, db += sum g.
 *   BATCH statistics of the batch itself (training, [P1] section 4): var is the
 *         biased batch variance and the statistics depend on the input.
 *   FIXED stored statistics (Caffe's use_global_stats, [P5] Backward_cpu; Darknet's
 *         rolling mean and variance when not training, [P1] section 4): the mean
 *         and variance are constants, so BN is a per-channel affine map and
 *         dz = gamma/sqrt(var + eps) * g; dgamma += sum g * x_norm; dbeta += sum g.
 *         var is the stored variance and x_norm the forward's normalised value. */
typedef enum cbb_bn_mode { CBB_BN_NONE = 0, CBB_BN_BATCH = 1, CBB_BN_FIXED = 2 } cbb_bn_mode;

/* Geometry of one convolutional block: Darknet layer fields batch, c, h, w
 * (input), n (out_c), size, stride, pad, batch_normalize, activation, groups,
 * dilation ([P3] layer struct).  Output size
 * out = (in + 2 pad - dilation (ksize - 1) - 1) / stride + 1, which is
 * im2col_cpu's (in + 2 pad - ksize) / stride + 1 ([P1] section 3.2) at dilation 1.
 * Groups ([P1] section 3.1, l.groups): group j owns output channels
 * [j out_c/groups, (j+1) out_c/groups), input channels [j in_c/groups, ...) and
 * weight block j; weights are [out_c][in_c/groups][ksize][ksize].  Dilation: tap
 * (kh, kw) of output (ho, wo) reads input (ho stride + kh dilation - pad,
 * wo stride + kw dilation - pad).  groups and dilation of 0 mean 1. */
typedef struct cbb_conv_desc {
  int32_t batch, in_c, in_h, in_w;
  int32_t out_c, ksize, stride, pad;
  int32_t batch_normalize; /* cbb_bn_mode; with BN its shift absorbs the conv bias      */
  int32_t act;             /* cbb_act                                                  */
  float slope;             /* leaky slope (0.1 in every page's network)                 */
  float bn_eps;            /* added to the variance inside the square root (1e-5)       */
  int32_t groups;          /* divides in_c and out_c                                    */
  int32_t dilation;        /* 1..16                                                      */
} cbb_conv_desc;

int cbb_abi_version(void);
/* Static text for a status code, or the last HIP error text for CBB_EHIP. */
const char* cbb_status_string(int status);
const char* cbb_last_error(void);

/* Device-side failure detection.  Host checks cover every argument error (the
 * asserts / CHECKs of the pages become status codes); a condition only the data
 * reveals is raised by the kernel that meets it as a bit in a per-GPU error word:
 *   CBB_DEVERR_LABEL  a softmax-loss label outside [0, classes) ([P2] layer 9).
 * cbb_get_device_error waits for `stream` (a host synchronisation, unlike every
 * other call), stores in *code the OR of the bits raised on the current GPU since
 * the previous query (0: none), and clears the word.  Kernels of other streams
 * still running on that GPU may raise bits after the read.  CBB_EINVAL when code
 * is NULL; CBB_EHIP when the wait or the read fails. */
#define CBB_DEVERR_LABEL 1
int cbb_get_device_error(void* stream, int* code);

/* Tracing: fn(user, kernel, stream) is called on the calling thread right after
 * each kernel the library enqueues (kernel = its name, stream = the hipStream_t
 * it went to), e.g. to record a HIP event after it.  Process-wide; NULL removes
 * the hook.  A hook must not call back into the library.  Always CBB_OK. */
typedef void (*cbb_launch_hook)(void* user, const char* kernel, void* stream);
int cbb_set_launch_hook(cbb_launch_hook fn, void* user);

/* ----------------------------------------------------------------------------
 * Conv block backward: backward_convolutional_layer of [P1] section 3.1 with
 * backward_batchnorm_layer of [P1] section 4:
 *   g      = delta * act'(y)                                 (gradient_array)
 *   BN:    dbeta += sum g;  dgamma += sum g * x_norm;        (backward_bias/_scale)
 *          BATCH: dz = gamma/sqrt(var+eps) * (g - mean(g) - x_norm * mean(g * x_norm))
 *          (the closed form of Caffe's BatchNormLayer Backward_cpu, [P5], after
 *           Darknet's scale_bias by gamma; means over batch and space)
 *          FIXED: dz = gamma/sqrt(var+eps) * g   (see cbb_bn_mode)
 *   no BN: db += sum g;  dz = g
 *   dw[o,i,kh,kw] += sum_{n,ho,wo} dz[n,o,ho,wo] * x[n,i,ho*s+kh-p,wo*s+kw-p]
 *   dx[n,i,h,w]   (+)= sum over (o,kh,kw) with h = ho*s+kh-p, w = wo*s+kw-p of
 *                      W[o,i,kh,kw] * dz[n,o,ho,wo]    (W^T x delta, then col2im)
 * Padding taps read zero.
 *
 * Arguments (shapes with N = batch, C = in_c, O = out_c, OH x OW the output):
 *   x       [N,C,H,W]     block input (net.input)
 *   w       [O,C/groups,k,k] weights
 *   y       [N,O,OH,OW]   activation output (l.output); NULL allowed iff act = LINEAR
 *   x_norm  [N,O,OH,OW]   normalised conv output (l.x_norm)   } required iff
 *   var     [O]           variance: biased batch variance     } batch_normalize,
 *                         (l.variance) or the stored one      } NULL otherwise
 *   gamma   [O]           BN scale (l.scales)                 }
 *   delta   [N,O,OH,OW]   dL/dy (l.delta on entry), read only
 *   dz      [N,O,OH,OW]   receives dL/dz (l.delta on exit); may equal delta
 *                         (in place).  NULL when act = LINEAR and no BN (dz is
 *                         delta itself), or to leave dz unstored on a layer for
 *                         which cbb_conv_fused_weights_data returns 1, with dx
 *                         given and x, delta, y, x_norm 16-byte aligned: the
 *                         fused dW + dX kernel then forms dz from
 *                         delta, y and x_norm as it stages them, and the
 *                         separate pass that writes dz, and its re-read, go
 *                         away.  Any other NULL dz is CBB_EINVAL.
 *   dw      [O,C/groups,k,k] += weight gradient (l.weight_updates)
 *   db      [O]           += bias gradient (l.bias_updates; with BN this is dbeta)
 *   dgamma  [O]           += scale gradient (l.scale_updates); BN only, else NULL
 *   dx      [N,C,H,W]     input gradient (net.delta); NULL skips it
 *   dx_accumulate         1: dx += ...; 0: dx = ...
 *   workspace             device scratch of at least cbb_conv_block_workspace_size
 *                         bytes, 256-byte aligned; contents on entry ignored.
 * Supported: 1 <= ksize <= 7, 1 <= stride <= 4, 0 <= pad <= dilation (ksize - 1),
 * all sizes whose element counts fit in int32 per tensor index and int64 overall.
 * Grouped or dilated layers run all groups in one launch (the group index on
 * the grid's y axis): the general implicit-GEMM kernels, except that grouped
 * undilated 3x3 pad-1 layers with in_c/groups a multiple of 32 and
 * out_c/groups a multiple of 64 take the row-streaming 3x3 weight-gradient
 * kernel, grouped undilated 3x3 pad-1 layers with in_c/groups a multiple of 32
 * and out_c/groups a multiple of 8 (16 at stride 2) take the tile-direct 3x3
 * input-gradient kernel, and depthwise layers (groups = in_c = out_c) take
 * streaming kernels.
 * ------------------------------------------------------------------------- */
int cbb_conv_block_workspace_size(const cbb_conv_desc* desc, size_t* bytes);
int cbb_conv_block_backward(const cbb_conv_desc* desc, const float* x, const float* w,
                            const float* y, const float* x_norm, const float* var,
                            const float* gamma, const float* delta, float* dz, float* dw,
                            float* db, float* dgamma, float* dx, int dx_accumulate,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Two consecutive blocks of a network ([P3] backward_network: layer i's input
 * gradient is layer i-1's delta; [P1] section 4: a block's act/BN backward first
 * sums g = delta * act'(y) and g * x_norm over its batch) can share a pass: the
 * kernel that writes the upper block's dx can add up the lower block's two sums
 * as it stores each element, so the lower block's call needs no reduction pass
 * over its delta.  Zero-initialise, then set:
 *   sums          this block's act/BN sums, produced by the call of the block above
 *                 it (its below_sums): float2 per output channel, (sum g,
 *                 sum g * x_norm) over the batch.  Batch-statistics BN only
 *                 (else CBB_EINVAL).  NULL: computed here.
 *   below_sums    receives the act/BN sums of the block below this one (whose delta
 *                 is this call's dx): float2 per input channel, as above.  Needs dx.
 *   below_y       that block's activation output [N,C,H,W] (NULL iff below_act is
 *                 LINEAR) and normalised conv output below_x_norm [N,C,H,W];
 *   below_act     its activation and leaky slope below_slope;
 *   below_apply_act  1: dx is left holding g = dx * act'(below_y) itself, the value
 *                 the block below's activation step turns its delta into ([P1]
 *                 sections 3.1 and 7: gradient_array scales the delta in place), so
 *                 that block's call can run with a LINEAR activation and read no y;
 *                 0: dx as without options.  Only 0 or 1, and 1 only with
 *                 below_sums.
 * The sums are over dx as the call leaves it (after dx_accumulate).  Where dx is
 * written by the stride-2 3x3 kernel over one 32-channel block (16-byte aligned,
 * width a multiple of 4) the sums are added up in its epilogue; otherwise a
 * reduction pass over dx follows (and, with below_apply_act, a pass that scales dx
 * in place).  Results equal those of separate calls up to the order of the
 * summation. */
typedef struct cbb_block_opts {
  const float* sums;
  float* below_sums;
  const float* below_y;
  const float* below_x_norm;
  int32_t below_act;
  float below_slope;
  int32_t below_apply_act;
} cbb_block_opts;

/* cbb_conv_block_backward with options (opts NULL: the same call); the same
 * workspace size.  CBB_EINVAL for options that break the rules above. */
int cbb_conv_block_backward_ex(const cbb_conv_desc* desc, const float* x, const float* w,
                               const float* y, const float* x_norm, const float* var,
                               const float* gamma, const float* delta, float* dz, float* dw,
                               float* db, float* dgamma, float* dx, int dx_accumulate,
                               const cbb_block_opts* opts, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------------------
 * The conv block backward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * cbb_conv_block_backward with the same arguments, results and errors, except that
 * its scratch memory is a static device buffer of CBB_NOALLOC_SCRATCH_BYTES that
 * the library owns (one per GPU, held from the library's load until the process
 * ends) instead of a workspace argument.  It allocates nothing and calls no
 * allocating routine.  The first call on a GPU looks up that GPU's buffer.
 * CBB_ESCRATCH, before any HIP call, when cbb_conv_block_workspace_size exceeds
 * the buffer (64 MiB holds every layer of the five workloads the library is
 * measured on).  Every call on a GPU shares that GPU's buffer, so calls that
 * overlap on one GPU (several streams or host threads) race: serialise them.
 * The buffer keeps whatever the last call left; no call relies on its contents.
 * ------------------------------------------------------------------------- */
#define CBB_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)
int cbb_conv_block_backward_noalloc(const cbb_conv_desc* desc, const float* x, const float* w,
                                    const float* y, const float* x_norm, const float* var,
                                    const float* gamma, const float* delta, float* dz, float* dw,
                                    float* db, float* dgamma, float* dx, int dx_accumulate,
                                    void* stream);

/* ----------------------------------------------------------------------------
 * Conv block forward: the tensors the backward reads, computed on the device
 * (forward_convolutional_layer of [P1] sections 3.1-3.2 with forward_batchnorm_layer
 * of [P1] section 4 and the *_activate functions of section 7):
 *   z = conv(x, W)  (+ bias[o] when batch_normalize = NONE; NULL bias = 0)
 *   BATCH: mean[o] = mean of z over (batch, space), var[o] = E[(z - mean)^2] (biased),
 *          both written;  FIXED: mean, var read (stored statistics)
 *   x_norm = (z - mean)/sqrt(var + eps),  u = gamma x_norm + beta  (BN),  u = z (no BN)
 *   y = act(u)
 * Shapes as in cbb_conv_block_backward; with BN, x_norm, mean, var, gamma, beta are
 * required and bias must be NULL (the BN shift absorbs it); without BN they must
 * be NULL.  y and x_norm must not overlap x or each other.  Workspace: at least
 * cbb_conv_block_forward_workspace_size bytes, 256-byte aligned.  The rolling
 * averages Darknet / Caffe keep for inference are not updated.
 * ------------------------------------------------------------------------- */
int cbb_conv_block_forward_workspace_size(const cbb_conv_desc* desc, size_t* bytes);
int cbb_conv_block_forward(const cbb_conv_desc* desc, const float* x, const float* w,
                           const float* bias, const float* gamma, const float* beta, float* mean,
                           float* var, float* x_norm, float* y, void* workspace,
                           size_t workspace_bytes, void* stream);

/* The three stages of cbb_conv_block_backward as separate calls (Caffe splits
 * the same work into backward_cpu_bias / weight_cpu_gemm / backward_cpu_gemm,
 * [P4] BaseConvolutionLayer).  Enqueued one after another on one stream with
 * the same workspace they do exactly what cbb_conv_block_backward does.
 * Each takes the workspace sized by cbb_conv_block_workspace_size.
 *
 * Stage 1, activation gradient + BN backward (or the bias sum):
 *   arguments as in cbb_conv_block_backward; writes dz (unless act = LINEAR
 *   without BN, where dz may be NULL and nothing is written), adds to db and
 *   (BN) dgamma. */
int cbb_conv_act_bn_backward(const cbb_conv_desc* desc, const float* y, const float* x_norm,
                             const float* var, const float* gamma, const float* delta, float* dz,
                             float* db, float* dgamma, void* workspace, size_t workspace_bytes,
                             void* stream);
/* Stage 2, weight gradient: dw [O,C,k,k] += dz (x) im2col(x)^T, from
 * dz [N,O,OH,OW] and x [N,C,H,W]. */
int cbb_conv_backward_weights(const cbb_conv_desc* desc, const float* x, const float* dz,
                              float* dw, void* workspace, size_t workspace_bytes, void* stream);
/* Stage 3, input gradient: dx [N,C,H,W] (+)= col2im(W^T dz).  dx must not
 * overlap w, dz or the workspace. */
int cbb_conv_backward_data(const cbb_conv_desc* desc, const float* w, const float* dz, float* dx,
                           int dx_accumulate, void* workspace, size_t workspace_bytes,
                           void* stream);
/* Stage 3 with the act/BN sums of the block below (cbb_block_opts: below_sums,
 * below_y, below_x_norm, below_act, below_slope, below_apply_act; sums must be NULL), the same
 * workspace size. */
int cbb_conv_backward_data_ex(const cbb_conv_desc* desc, const float* w, const float* dz,
                              float* dx, int dx_accumulate, const cbb_block_opts* opts,
                              void* workspace, size_t workspace_bytes, void* stream);
/* 1 when the input-gradient kernel of this layer adds up the act/BN sums of the
 * block below in its epilogue (cbb_block_opts, given 16-byte aligned tensors and
 * a width that is a multiple of 4); 0 when a reduction pass over dx follows
 * instead; a negative status for a bad descriptor. */
int cbb_conv_fuses_below_sums(const cbb_conv_desc* desc);
/* Stages 2 and 3 together (the two GEMMs of [P1] section 3.1 that read the
 * same delta): dw += weight gradient and, when dx is not NULL, dx (+)= input
 * gradient, with the meanings and buffers of the two calls above.  For the
 * layers cbb_conv_fused_weights_data reports, both come from one kernel that
 * reads dz once; otherwise this is stage 2 followed by stage 3.  dx must not
 * overlap x, w, dz, dw or the workspace. */
int cbb_conv_backward_weights_data(const cbb_conv_desc* desc, const float* x, const float* w,
                                   const float* dz, float* dw, float* dx, int dx_accumulate,
                                   void* workspace, size_t workspace_bytes, void* stream);
/* 1 when cbb_conv_backward_weights_data (and cbb_conv_block_backward with dx)
 * computes dW and dX in one fused kernel for this descriptor: 3x3 kernel, pad 1,
 * stride 1, at most 3 input and at most 32 output channels, input width a
 * multiple of 4 (a first layer on an RGB image), provided x and dz are 16-byte
 * aligned at the call; 0 otherwise; a negative status for an invalid
 * descriptor.  Informational: the results do not depend on it. */
int cbb_conv_fused_weights_data(const cbb_conv_desc* desc);
/* 1 when cbb_conv_block_backward, on this descriptor with batch statistics, forms dz
 * inside the weight-gradient kernel: 3x3, pad 1, stride 1 or 2, 32 input channels,
 * output channels a multiple of 64, widths multiples of 4, provided x,
 * delta, y, x_norm and dz are 16-byte aligned and dz is none of delta, y, x_norm at the
 * call.  That kernel then computes dz from delta, y and x_norm with the per-channel map
 * of the BN backward while it stages them and writes dz for the input gradient, so the
 * separate pass that writes dz goes away (dz is still written).  0 otherwise; a
 * negative status for an invalid descriptor.  Informational: the results do not
 * depend on it. */
int cbb_conv_dw_forms_dz(const cbb_conv_desc* desc);

/* Activation gradient alone (gradient_array, [P1] sections 3.1 and 7):
 * g[i] = delta[i] * act'(y[i]) for i < count.  g may equal delta. */
int cbb_act_backward(int act, float slope, const float* y, const float* delta, float* g,
                     int64_t count, void* stream);

/* Batch-norm backward alone (training statistics), from g = dL/du where
 * u = gamma * x_norm + beta; tensors [n, c, hw]:
 *   dbeta += sum g;  dgamma += sum g * x_norm;
 *   dz = gamma/sqrt(var+eps) * (g - mean(g) - x_norm * mean(g * x_norm)).
 * ([P1] section 4 backward_batchnorm_layer; [P5] Backward_cpu.)  dz may equal g. */
int cbb_bn_backward_workspace_size(int n, int c, int64_t hw, size_t* bytes);
int cbb_bn_backward(int n, int c, int64_t hw, float eps, const float* g, const float* x_norm,
                    const float* var, const float* gamma, float* dz, float* dgamma, float* dbeta,
                    void* workspace, size_t workspace_bytes, void* stream);
/* The same with fixed (stored) statistics, see CBB_BN_FIXED:
 *   dbeta += sum g;  dgamma += sum g * x_norm;  dz = gamma/sqrt(var+eps) * g.
 * ([P5] Backward_cpu with use_global_stats, which divides the top gradient by
 * sqrt(var + eps), after Darknet's scale_bias by gamma.)  Same workspace size as
 * cbb_bn_backward; dz may equal g. */
int cbb_bn_backward_fixed(int n, int c, int64_t hw, float eps, const float* g,
                          const float* x_norm, const float* var, const float* gamma, float* dz,
                          float* dgamma, float* dbeta, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Inner-product backward ([P2] layer 8), batch M, in K, out N:
 *   dw [N,K] += delta^T [N,M] x [M,K];  db [N] += sum over the batch of delta;
 *   dx [M,K] (+)= delta [M,N] x w [N,K]   (NULL skips; dx_accumulate as above).
 * db may be NULL (no bias term). */
int cbb_fc_backward(int batch, int in_dim, int out_dim, const float* x, const float* w,
                    const float* delta, float* dw, float* db, float* dx, int dx_accumulate,
                    void* stream);

/* Softmax-with-loss gradient ([P2] layer 9): dlogits = prob, minus 1 at each
 * sample's label, times loss_weight / batch (one label per sample, so the
 * normalised count and the outer count are both `batch`).  prob, dlogits
 * [batch, classes]; labels int32 [batch].  A label outside [0, classes)
 * leaves its row without the -1, adds 1 to *bad_labels (device int32, may be
 * NULL; a count the caller reads when it wants to) and raises
 * CBB_DEVERR_LABEL in the GPU's error word (cbb_get_device_error).  The
 * pages store labels as floats and cast them to int ([P2] layer 9), so a bad
 * value is a property of the data that only the kernel sees. */
int cbb_softmax_loss_backward(int batch, int classes, const float* prob, const int32_t* labels,
                              float loss_weight, float* dlogits, int32_t* bad_labels,
                              void* stream);

/* The loss gradient above followed by the backward of the inner product that
 * produced the logits ([P2] layers 9 and 8 together): dlogits as above, then
 * dw [classes, in_dim] += dlogits^T x, db [classes] += sum dlogits,
 * dx [batch, in_dim] = dlogits x w (NULL skips). */
int cbb_fc_softmax_backward(int batch, int in_dim, int classes, const float* prob,
                            const int32_t* labels, float loss_weight, const float* x,
                            const float* w, float* dlogits, float* dw, float* db, float* dx,
                            int32_t* bad_labels, void* stream);

/* Softmax backward along the channel axis ([P4] SoftmaxLayer Backward_cpu):
 * tensors [outer, channels, inner] (inner = 1 for [batch, classes] rows),
 *   dx[i,c,k] = (dy[i,c,k] - sum_c' dy[i,c',k] * y[i,c',k]) * y[i,c,k]
 * with y the softmax output.  dx may equal dy, not y.  (cbb_softmax_loss_backward
 * is this composed with the cross-entropy gradient, in closed form.) */
int cbb_softmax_backward(int outer, int channels, int64_t inner, const float* y, const float* dy,
                         float* dx, void* stream);

/* Shortcut backward for equal shapes ([P1] section 5): d_main += alpha*delta
 * (axpy into the previous layer's delta); d_from += beta*delta (shortcut_cpu
 * with s1 = 1, s2 = beta, into the source layer's delta).  d_main and d_from
 * must not overlap each other or delta. */
int cbb_shortcut_backward(int64_t count, float alpha, float beta, const float* delta,
                          float* d_main, float* d_from, void* stream);

/* Shortcut backward between layers of different shapes ([P1] section 5,
 * shortcut_cpu): delta is [batch, c1, h1, w1] (the shortcut's output), d_from
 * [batch, c2, h2, w2] (the source layer's delta).  With stride = w1/w2 and
 * sample = w2/w1 (each raised to at least 1), over k < min(c1,c2),
 * j < min(h1,h2), i < min(w1,w2):
 *   d_from[b, k, j*sample, i*sample] += beta * delta[b, k, j*stride, i*stride]
 * and, unless d_main is NULL, d_main [batch, c1, h1, w1] += alpha * delta.
 * CBB_ESHAPE when w1/w2 != h1/h2 or w2/w1 != h2/h1 (the page's asserts).
 * With equal shapes this is cbb_shortcut_backward. */
int cbb_shortcut_backward_resize(int batch, int w1, int h1, int c1, int w2, int h2, int c2,
                                 float alpha, float beta, const float* delta, float* d_main,
                                 float* d_from, void* stream);

/* Route backward ([P1] section 6): the route delta holds, per image, the
 * inputs' outputs one after another (in_sizes[t] floats each, t < n_in <= 8);
 * for every input t and image j, d_in[t][j*in_sizes[t] + e] += the matching
 * route-delta element.  `in_sizes` and `d_in` are HOST arrays (d_in of device
 * pointers). */
int cbb_route_backward(int batch, int n_in, const int64_t* in_sizes, const float* delta,
                       float* const* d_in, void* stream);

/* Nearest-neighbour upsample backward (adjoint of y[h,w] = x[h/scale, w/scale];
 * the pages name the layer but do not show it):
 *   dx[n,c,h,w] += sum_{a,b < scale} delta[n,c,h*scale+a,w*scale+b];
 * dx [n,c,h,w], delta [n,c,h*scale,w*scale]. */
int cbb_upsample_backward(int n, int c, int h, int w, int scale, const float* delta, float* dx,
                          void* stream);

/* Max-pool backward ([P2] layer 5): dx = 0, then every pooled output adds
 * its delta at the bottom pixel its mask names.  Window ksize x ksize,
 * stride `stride`, no padding: oh = (ih - ksize)/stride + 1.  idx int32
 * [n,c,oh,ow] holds the per-plane flat index h*iw + w of the winner, which
 * must lie inside that output's window (as a max-pool forward produces);
 * dx [n,c,ih,iw] is overwritten. */
int cbb_maxpool_backward(int n, int c, int ih, int iw, int ksize, int stride,
                         const int32_t* idx, const float* delta, float* dx, void* stream);

/* Parameter update after a full batch (update_network -> l.update(layer, batch,
 * learning_rate, momentum, decay), called once (seen / batch) % subdivisions == 0,
 * [P1] section 1; [P3] layer struct: the update hook and the weight_updates buffer
 * it consumes).  The pages print no formula;
 * this is gradient descent with momentum and L2 weight decay in which the
 * accumulated-gradient buffer doubles as the momentum buffer (the next backward
 * adds onto it, as every parameter gradient here accumulates):
 *   u = dw + decay * batch * w;   w -= (learning_rate / batch) * u;   dw = momentum * u
 * for i < n.  dw holds the gradient summed over the batch (dw, db, dgamma of the
 * calls above); pass decay = 0 for biases and BN scales.  w and dw device arrays
 * of n floats that do not overlap.  CBB_EINVAL for a negative size or rate,
 * batch < 1 or NULL pointers. */
int cbb_sgd_update(int64_t n, int batch, float learning_rate, float momentum, float decay,
                   float* w, float* dw, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CBB_H */
