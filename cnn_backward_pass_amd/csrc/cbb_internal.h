// cbb_internal.h -- shared device/host helpers of libcbb (gfx950 only).
//
// The fp32 matrix-core tile used by every contraction in the library lives
// here.  Operand lane layouts of the gfx950 fp32 MFMA instructions (checked on
// the device by a lane-tagging probe):
//   v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][l/32] and B[l/32][l%32];
//     accumulator register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/cbb.h"

namespace cbb {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;  // every kernel runs 4 waves of 64 lanes

// Geometry of one convolution, derived from cbb_conv_desc.  With groups, the
// general kernels run once per group on a geometry whose C and OC are the
// group's channel counts while xs / zs keep the image strides of the whole
// tensors; everywhere else xs = C*HW and zs = OC*OHW.
struct ConvGeom {
  int N, C, H, W, OC, K, S, P, OH, OW;
  int HW, OHW, J;  // J = C*K*K, columns of the weight-gradient matrix
  int64_t Q;       // N*OH*OW, the reduction length of the weight gradient
  int G, D;        // groups, dilation (tap k reads input row ho*S + k*D - P)
  int64_t xs, zs;  // image strides (floats) of x / dx and of dz
  // offsets (floats) from one group to the next: x / dx channels, dz channels, and
  // weight / dW blocks; the general kernels take the group from blockIdx.y
  int64_t gx, gz, gw;
};

// Host-side launch bookkeeping -------------------------------------------------
void set_hip_error(hipError_t e, const char* where);
const char* last_error_text();
// After a kernel is enqueued: note_launch calls the launch hook (cbb_set_launch_hook)
// with the kernel's name; check_error records a pending HIP error; check_launch does
// both (CBB_OK or CBB_EHIP).
void note_launch(const char* kernel, hipStream_t st);
int check_error(const char* where);
int check_launch(const char* where, hipStream_t st);
// The argument rules of cbb_conv_block_backward other than the workspace's
// (CBB_OK or the status the call returns), checked before any HIP call.
int check_block_backward(const cbb_conv_desc* desc, const float* x, const float* w,
                         const float* y, const float* x_norm, const float* var,
                         const float* gamma, const float* delta, const float* dz,
                         const float* dw, const float* db, const float* dgamma, const float* dx,
                         int dx_accumulate);
// This device's error word (CBB_DEVERR_* bits, read by cbb_get_device_error), or
// nullptr with the HIP error recorded.
int32_t* device_error_word();

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Wave-level fp32 sum of one value per lane (fixed butterfly: deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Block-level sum of one value per thread for 256-thread blocks; every thread
// gets the total.  `scratch` needs 4 floats of LDS.
__device__ __forceinline__ float block_sum_256(float v, float* scratch) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  return (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
}

// ---------------------------------------------------------------------------
// MFMA tile core.
//
// A work-group of 4 waves computes a BM x BN block of C = A x B over a range of
// the reduction index.  Waves are arranged WM x WN x WK (WM*WN*WK = 4): each
// wave owns RM x RN blocks of 32 x 32 (one 32x32x2 accumulator each, so a wave
// tile is 32RM x 32RN) and, when WK > 1, a share of every K tile, with the WK
// partial blocks summed through LDS at the end.  K tiles are BK = 32*WK*KSUB
// deep and staged in LDS, double-buffered, as
//   As[BK][BM + 1]  (A transposed: K-major, padded against bank conflicts)
//   Bs[BK][BN + 1]
// The loaders (supplied by each kernel) fill registers for tile t+2 while the
// matrix cores work on tile t.
// ---------------------------------------------------------------------------
template <int WM_, int WN_, int WK_, int KSUB_ = 1, int RM_ = 1, int RN_ = 1>
struct TileShape {
  static constexpr int WM = WM_, WN = WN_, WK = WK_, KSUB = KSUB_, RM = RM_, RN = RN_;
  static_assert(WM * WN * WK == 4, "4 waves per work-group");
  // each wave consumes KSUB slabs of 32 K rows per tile
  static constexpr int BM = 32 * WM * RM, BN = 32 * WN * RN, BK = 32 * WK * KSUB;
  static constexpr int LDA = BM + 1, LDB = BN + 1;
  static constexpr int A_PER_T = BM * BK / kThreads;  // A elements each thread stages
  static constexpr int B_PER_T = BN * BK / kThreads;
  static constexpr int BUF_FLOATS = BK * LDA + BK * LDB;  // one stage (A and B tiles)
  static constexpr int LDS_FLOATS = 2 * BUF_FLOATS;        // double-buffered
  static constexpr int NACC = RM * RN;
  static constexpr int RED_FLOATS = (WK - 1) * WM * WN * NACC * 64 * 16;
  static_assert(RED_FLOATS <= LDS_FLOATS, "WK reduction reuses the staging area");
};

template <class TS>
struct Acc {
  f32x16 v[TS::RM][TS::RN];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TS::RM; ++i)
#pragma unroll
      for (int j = 0; j < TS::RN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[i][j][r] = 0.f;
  }
};

// Row offset (within the block tile) of accumulator (i, j)'s 32x32 block for wave (wm, wn).
template <class TS>
__device__ __forceinline__ int acc_m0(int wm, int i) { return (wm * TS::RM + i) * 32; }
template <class TS>
__device__ __forceinline__ int acc_n0(int wn, int j) { return (wn * TS::RN + j) * 32; }

// One K tile of MFMA work for the calling wave: 16*KSUB steps of K = 2 over the
// wave's K rows [wk*32*KSUB, (wk+1)*32*KSUB).  All operand fragments are read
// from LDS first and the matrix-core chain is issued afterwards, so the LDS
// latency is paid once per 32 K rows instead of once per step.
template <class TS>
__device__ __forceinline__ void mfma_tile(const float* __restrict__ As, const float* __restrict__ Bs,
                                          Acc<TS>& acc, int wm, int wn, int wk, int lane) {
  const int col = lane & 31, khalf = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < TS::KSUB; ++ks) {
    const int krow = (wk * TS::KSUB + ks) * 32 + khalf;
    float fa[TS::RM][16], fb[TS::RN][16];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
#pragma unroll
      for (int i = 0; i < TS::RM; ++i)
        fa[i][kk] = As[(krow + 2 * kk) * TS::LDA + acc_m0<TS>(wm, i) + col];
#pragma unroll
      for (int j = 0; j < TS::RN; ++j)
        fb[j][kk] = Bs[(krow + 2 * kk) * TS::LDB + acc_n0<TS>(wn, j) + col];
    }
    // keep the scheduler from sinking the reads back between the matrix-core steps
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int i = 0; i < TS::RM; ++i)
#pragma unroll
        for (int j = 0; j < TS::RN; ++j)
          acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][kk], fb[j][kk], acc.v[i][j], 0,
                                                             0, 0);
  }
}

// Double-buffered main loop over K tiles [kbeg, kend) in steps of BK.
//   load(k0)   : global -> registers for the tile starting at k0 (may be any k0 < kend)
//   store(buf) : registers -> LDS stage `buf` (A at buf, B at buf + BK*LDA)
// Per tile t: the matrix cores consume stage t%2 while stage (t+1)%2 receives
// tile t+1 and the loads of tile t+2 are in flight; one barrier per tile.
template <class TS, class Load, class Store>
__device__ __forceinline__ void gemm_mainloop(float* lds, int64_t kbeg, int64_t kend, Load&& load,
                                              Store&& store, Acc<TS>& acc, int wm, int wn, int wk,
                                              int lane) {
  if (kbeg >= kend) return;
  load(kbeg);
  store(lds);
  if (kbeg + TS::BK < kend) load(kbeg + TS::BK);
  __syncthreads();
  int cur = 0;
  for (int64_t k0 = kbeg;; k0 += TS::BK) {
    const float* A = lds + cur * TS::BUF_FLOATS;
    mfma_tile<TS>(A, A + TS::BK * TS::LDA, acc, wm, wn, wk, lane);
    if (k0 + TS::BK >= kend) break;
    store(lds + (cur ^ 1) * TS::BUF_FLOATS);
    if (k0 + 2 * TS::BK < kend) load(k0 + 2 * TS::BK);
    __syncthreads();
    cur ^= 1;
  }
}

// Sum the WK partial accumulators of a work-group into the wk == 0 waves.
// Uses `red` (LDS; the staging area is large enough) after a barrier.  All
// threads must call it.
template <class TS>
__device__ __forceinline__ void reduce_wk(Acc<TS>& acc, float* red, int wm, int wn, int wk,
                                          int lane) {
  if constexpr (TS::WK > 1) {
    __syncthreads();
    const int slot = (wm + TS::WM * wn) * TS::NACC;
    if (wk > 0) {
      float* dst = red + ((wk - 1) * TS::WM * TS::WN * TS::NACC + slot) * 64 * 16 + lane;
#pragma unroll
      for (int i = 0; i < TS::RM; ++i)
#pragma unroll
        for (int j = 0; j < TS::RN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[((i * TS::RN + j) * 16 + r) * 64] = acc.v[i][j][r];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int q = 1; q < TS::WK; ++q) {
        const float* src = red + ((q - 1) * TS::WM * TS::WN * TS::NACC + slot) * 64 * 16 + lane;
#pragma unroll
        for (int i = 0; i < TS::RM; ++i)
#pragma unroll
          for (int j = 0; j < TS::RN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc.v[i][j][r] += src[((i * TS::RN + j) * 16 + r) * 64];
      }
    }
  }
}

// Work-groups are dispatched round-robin over the 8 XCDs, each with its own L2.
// Remap the dispatch index so that XCD x runs one contiguous range of logical
// work-group ids: logical neighbours (tiles that read the same operands) then
// share an L2 instead of being spread over eight.  A bijection on [0, n).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_remap(int phys, int n) {
  const int per = n / kXcds, rem = n % kXcds;
  const int xcd = phys % kXcds, k = phys / kXcds;
  return xcd * per + min(xcd, rem) + k;
}

// LDS address of a shared-memory float, as the direct global-to-LDS copy builtin
// takes it (the copy of a wave fills 64 consecutive 4- or 16-byte slots from there).
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(float* p) {
  return (__attribute__((address_space(3))) void*)p;
}

// Row / column of accumulator register r of lane `lane` inside a wave's 32x32 block.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// Kernel launchers (host), one per translation unit's kernels ------------------
// Split-K partial sums are added in groups of this many, in a fixed order.
constexpr int kReduceGroup = 32;
// dw += the ordered sum of `splits` partial weight gradients in ws ([split][o][i][tap],
// or tap-major [split][tap][o][i] when tapmajor); two levels when groups > 0.
int launch_dw_reduce(const ConvGeom& g, float* dw, float* ws, int splits, int groups,
                     int tapmajor, hipStream_t st);
// Depthwise convolution (groups = in_c = out_c): streaming per-channel kernels.
bool conv_depthwise(const ConvGeom& g);
size_t conv_depthwise_workspace(const ConvGeom& g);
int launch_depthwise_dw(const ConvGeom& g, const float* x, const float* dz, float* dw, float* ws,
                        hipStream_t st);
int launch_depthwise_dx(const ConvGeom& g, const float* wt, const float* dz, float* dx,
                        int accumulate, hipStream_t st);
// 1x1 stride-1 gradients with direct global-to-LDS staging (16-byte aligned operands).
bool conv1x1_dma_ok(const ConvGeom& g, const void* a, const void* b);
size_t conv1x1_dw_workspace(const ConvGeom& g);
int launch_conv1x1_dw(const ConvGeom& g, const float* x, const float* dz, float* dw, float* ws,
                      hipStream_t st);
int launch_conv1x1_dx(const ConvGeom& g, const float* wt, const float* dz, float* dx,
                      int accumulate, hipStream_t st);
ConvGeom make_geom(const cbb_conv_desc& d);
size_t conv_dw_workspace(const ConvGeom& g);
int launch_conv_dw(const ConvGeom& g, const float* x, const float* dz, float* dw, float* ws,
                   hipStream_t st);
size_t conv_dx_workspace(const ConvGeom& g);
// Activation derivative read from the activation output y, as Darknet's
// *_gradient functions compute it ("YOLOv3 backpropagation", section 7).
__device__ __forceinline__ float act_grad(int act, float slope, float y) {
  switch (act) {
    case CBB_ACT_LEAKY: return y > 0.f ? 1.f : slope;
    case CBB_ACT_LOGISTIC: return (1.f - y) * y;
    case CBB_ACT_RELU: return y > 0.f ? 1.f : 0.f;
    case CBB_ACT_TANH: return 1.f - y * y;
    case CBB_ACT_ELU: return y >= 0.f ? 1.f : y + 1.f;
    case CBB_ACT_SELU: return y >= 0.f ? 1.0507f : y + 1.0507f * 1.6732f;
    case CBB_ACT_PLSE: return (y < 0.f || y > 1.f) ? .01f : .125f;
    case CBB_ACT_LHTAN: return (y > 0.f && y < 1.f) ? 1.f : .001f;
    case CBB_ACT_HARDTAN: return (y > -1.f && y < 1.f) ? 1.f : 0.f;
    case CBB_ACT_STAIR: return floorf(y) == y ? 0.f : 1.f;
    case CBB_ACT_RAMP: return (y > 0.f ? 1.f : 0.f) + .1f;
    case CBB_ACT_RELIE: return y > 0.f ? 1.f : .01f;
    case CBB_ACT_LOGGY: {
      const float s = (y + 1.f) * .5f;
      return 2.f * (1.f - s) * s;
    }
    default: return 1.f;
  }
}

// Activation of u (the forward's *_activate functions, "YOLOv3 backpropagation",
// section 7).
__device__ __forceinline__ float act_fwd(int act, float slope, float u) {
  switch (act) {
    case CBB_ACT_LEAKY: return u > 0.f ? u : slope * u;
    case CBB_ACT_LOGISTIC: return 1.f / (1.f + expf(-u));
    case CBB_ACT_RELU: return u > 0.f ? u : 0.f;
    case CBB_ACT_TANH: return tanhf(u);
    case CBB_ACT_ELU: return u >= 0.f ? u : expm1f(u);
    case CBB_ACT_SELU: return u >= 0.f ? 1.0507f * u : 1.0507f * 1.6732f * expm1f(u);
    case CBB_ACT_PLSE:
      if (u < -4.f) return .01f * (u + 4.f);
      if (u > 4.f) return .01f * (u - 4.f) + 1.f;
      return .125f * u + .5f;
    case CBB_ACT_LHTAN:
      if (u < 0.f) return .001f * u;
      if (u > 1.f) return .001f * (u - 1.f) + 1.f;
      return u;
    case CBB_ACT_HARDTAN: return u < -1.f ? -1.f : (u > 1.f ? 1.f : u);
    case CBB_ACT_STAIR: {
      const float n = floorf(u);
      return fmodf(n, 2.f) == 0.f ? floorf(u * .5f) : (u - n) + floorf(u * .5f);
    }
    case CBB_ACT_RAMP: return (u > 0.f ? u : 0.f) + .1f * u;
    case CBB_ACT_RELIE: return u > 0.f ? u : .01f * u;
    case CBB_ACT_LOGGY: return 2.f / (1.f + expf(-u)) - 1.f;
    default: return u;
  }
}
// (count, mean, M2 = sum of squared deviations) of a run of values, and the merge of
// two runs (Chan, Golub and LeVeque's update: mean = mean_a + d n_b / n,
// M2 = M2_a + M2_b + d^2 n_a n_b / n with d = mean_b - mean_a).
struct Moments {
  float n, mean, m2;
};
__device__ __forceinline__ Moments merge_moments(Moments a, Moments b) {
  if (b.n == 0.f) return a;
  if (a.n == 0.f) return b;
  const float n = a.n + b.n, d = b.mean - a.mean, fb = b.n / n;
  return Moments{n, a.mean + d * fb, a.m2 + b.m2 + d * d * a.n * fb};
}

bool conv_fused_dwdx_ok(const ConvGeom& g);
size_t conv_fused_workspace(const ConvGeom& g);
// dz of a block formed while it is staged instead of read back: with dz = delta,
// g = delta * act'(y) and the per-channel map of the BN backward,
//   dz[c] = coef[c] * g + coef[C + c] + coef[2C + c] * x_norm
// (y NULL: act linear; xn NULL: the third term is absent).
// The act/BN sums of the block below a convolution, added up by the kernel that
// writes this convolution's input gradient (the delta of that block): that
// block's y and x_norm (dx's shape; y may stand in for nothing under LINEAR) and
// activation.  The kernel writes partials part[c][nseg]; the launcher sets nseg
// (0: the route taken could not add them up, the caller reduces dx instead).
// Work-groups of the persistent stride-2 input-gradient kernel (two per CU), which
// also bounds the partials it writes for the block below.
constexpr int kDxS2pGroups = 2 * 256;
struct BnBelow {
  const float* y;
  const float* xn;
  int act;
  float slope;
  float2* part;
  int nseg;    // > 0: the input-gradient kernel wrote nseg partials per channel
  int apply;   // store g = dx * act'(y) in place of dx (the kernel does it when nseg > 0)
};
struct DzSource {
  const float* y;
  const float* xn;
  const float* coef;
  int act;
  float slope;
};
int launch_conv_fused_dwdx(const ConvGeom& g, const float* x, const float* wt, const float* dz,
                           float* dw, float* dx, int accumulate, float* ws, hipStream_t st,
                           const DzSource* src = nullptr);
bool conv_dw_forms_dz_ok(const ConvGeom& g);
int launch_conv_dw_forming_dz(const ConvGeom& g, const float* x, const float* delta,
                              const DzSource& src, float* dzout, float* dw, float* ws,
                              hipStream_t st);
int launch_conv_dx(const ConvGeom& g, const float* wt, const float* dz, float* dx, int accumulate,
                   float* ws, hipStream_t st, BnBelow* below = nullptr);
// Whether launch_conv_dx adds up the block below's act/BN sums in its kernel (given
// 16-byte aligned tensors at run time).
bool conv_dx_sums_below_ok(const ConvGeom& g);
size_t actbn_workspace(int N, int C, int64_t HW);
int launch_actbn(int N, int C, int64_t HW, const float* delta, const float* y, const float* xn,
                 int act, float slope, const float* var, const float* gamma, float eps, int bn,
                 float* dz, float* dgamma, float* dbeta_or_db, void* ws, hipStream_t st,
                 float* coef = nullptr, const float2* sums = nullptr);
// sums[c] = (sum g, sum g*x_norm) of a batch-statistics act/BN stage over its channel
// c (g = delta * act'(y)): a reduction pass into the partials in ws, then a fixed-
// order fold; launch_bn_sums_fold folds partials part[c][nseg] another kernel wrote.
size_t bn_sums_workspace(int N, int C, int64_t HW);
int launch_bn_sums(int N, int C, int64_t HW, const float* delta, const float* y, const float* xn,
                   int act, float slope, void* ws, float2* sums, hipStream_t st);
int launch_bn_sums_fold(const float2* part, int C, int nseg, float2* sums, hipStream_t st);
int launch_act_backward(int act, float slope, const float* y, const float* delta, float* g,
                        int64_t count, hipStream_t st);
int launch_bn_act_forward(int N, int C, int64_t HW, int bn, float eps, int act, float slope,
                          const float* gamma, const float* beta, float* mean, float* var,
                          float* xn, float* y, void* ws, hipStream_t st);
bool conv_dx_specialised(const ConvGeom& g);
size_t conv_forward_workspace(const ConvGeom& g, bool has_bias);
// The block forward of a short-reduction layer (C*K*K <= 32, at most 32 output channels)
// with BN in kernels that compute z again instead of storing it.
bool conv_forward_first_fused(const ConvGeom& g, int bn);
int launch_conv_block_forward_first(const ConvGeom& g, const float* x, const float* wt, int bn,
                                    float eps, int act, float slope, const float* gamma,
                                    const float* beta, float* mean, float* var, float* xn,
                                    float* y, float* ws, hipStream_t st);
int launch_conv_forward(const ConvGeom& g, const float* x, const float* wt, const float* bias,
                        float* z, float* ws, hipStream_t st);
int launch_shortcut(int64_t count, float alpha, float beta, const float* delta, float* d_main,
                    float* d_from, hipStream_t st);
int launch_shortcut_resize(int batch, int w1, int h1, int c1, int w2, int h2, int c2, float alpha,
                           float beta, const float* delta, float* d_main, float* d_from,
                           hipStream_t st);
int launch_softmax_backward(int outer, int channels, int64_t inner, const float* y,
                            const float* dy, float* dx, hipStream_t st);
int launch_route(int batch, int n_in, const int64_t* sizes, const float* delta,
                 float* const* d_in, hipStream_t st);
int launch_upsample(int n, int c, int h, int w, int scale, const float* delta, float* dx,
                    hipStream_t st);
int launch_maxpool(int n, int c, int ih, int iw, int k, int s, const int32_t* idx,
                   const float* delta, float* dx, hipStream_t st);
int launch_softmax_loss(int batch, int classes, const float* prob, const int32_t* labels,
                        float loss_weight, float* dlogits, int32_t* bad, hipStream_t st);
int launch_sgd_update(int64_t n, int batch, float lr, float momentum, float decay, float* w,
                      float* dw, hipStream_t st);
// C[m][n] (+)= sum_k A(m,k) B(k,n) on the fp32 matrix cores (layers.hip), `batch`
// problems with B and C offset by sbb / scb elements each.
struct GemmArgs {
  int M, N, K;
  const float* A;
  int64_t sam, sak;
  const float* B;
  int64_t sbk, sbn;
  float* C;
  int64_t ldc;
  int accumulate;
  int64_t sbb, scb;
};
int launch_gemm(const GemmArgs& a, hipStream_t st, int batch = 1);
int launch_fc(int batch, int in_dim, int out_dim, const float* x, const float* w,
              const float* delta, float* dw, float* db, float* dx, int dx_accumulate,
              hipStream_t st);

}  // namespace cbb
