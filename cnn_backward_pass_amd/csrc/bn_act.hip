// bn_act.hip -- activation gradient + batch-norm backward (or bias sum) as two
// streaming passes over the conv output, bandwidth-bound by design.
//
// "YOLOv3 backpropagation: full-flow source analysis" (suzhouguqin.com):
//   section 3.1 gradient_array: g = delta * act'(y), act' read from the output;
//   section 4 backward_batchnorm_layer: dbeta += sum g (backward_bias),
//   dgamma += sum g*x_norm (backward_scale_cpu), then the input gradient;
//   section 7: the *_gradient functions of the fourteen activations.
// "Understanding BatchNorm" (javaforall.cn): Caffe's closed form
//   dz = (g' - mean(g') - mean(g' x_norm) x_norm) / sqrt(var + eps), g' = gamma g.
//
// A channel small enough for one work-group (N*HW <= 24576 with BN, 40960
// without) takes one pass instead (actbn_channel): loads, sums, dz (or the map),
// all in registers.
// Pass 1 (actbn_reduce) : each work-group sums (g, g*x_norm) over one segment
//                         of one channel -> workspace partials[c][seg].  Without
//                         batch statistics dz does not depend on the sums and is
//                         written here (then actbn_fold adds the sums up).
// Pass 2 (actbn_apply)  : each work-group first folds its channel's partials in
//                         a fixed order (deterministic), derives the per-channel
//                         affine map dz = a*g + b + c*x_norm, writes dz for its
//                         segment; segment 0 also adds the channel's sums into
//                         dgamma / dbeta (or db).
// When a gradient kernel forms dz itself, actbn_coef replaces pass 2: one
// work-group per channel folds the sums and writes the map (a, b, c).
// The forward's statistics, normalisation and activation (bnf_*) follow below.
// A channel's data is N planes of HW floats, (n*C + c)*HW apart; a segment is a
// contiguous run of the flattened (n, hw) index.
#include "cbb_internal.h"

namespace cbb {

// The streaming kernels take the activation as a template argument for the four
// the networks use (no branch in the loop); kActAny takes it from `act_rt`.
constexpr int kActAny = -1;
// BN modes: none (bias sum), batch statistics, fixed statistics.
constexpr int kBnNone = 0, kBnBatch = 1, kBnFixed = 2;

// Work split of one channel: its N planes of HW floats are cut into `nseg`
// segments.  Large planes (HW >= kPlaneSplit) are cut into `parts` equal ranges
// per plane, one segment each; small planes are grouped `group` whole planes per
// segment.  A segment is thus a list of contiguous ranges inside planes, which
// a work-group streams with unrolled float4 accesses (no per-element index math).
constexpr int kPlaneSplit = 16384;

struct SegGeom {
  int N, C, HW;
  int64_t M;      // N*HW elements per channel
  int nseg;       // segments per channel
  int parts;      // ranges per plane (large planes), else 1
  int group;      // planes per segment (small planes), else 1
  int chunk;      // elements per range (multiple of 4 when VEC), large planes
};

// Visit segment `sg` of channel `c`: f(offset, vec4) for every element (VEC:
// every float4) of its ranges; thread t takes elements t, t+256, ... unrolled 4x.
template <bool VEC, class F>
__device__ __forceinline__ void for_segment(const SegGeom& s, int c, int sg, F&& f) {
  int n0, n1, r0, r1;
  if (s.parts > 1) {
    n0 = sg / s.parts;
    n1 = n0 + 1;
    const int part = sg - n0 * s.parts;
    r0 = part * s.chunk;
    r1 = min(s.HW, r0 + s.chunk);
  } else {
    n0 = sg * s.group;
    n1 = min(s.N, n0 + s.group);
    r0 = 0;
    r1 = s.HW;
    if (s.HW < 4 * kThreads) {
      // small planes: spread the threads over the segment's planes (all lanes busy)
      const int per = VEC ? s.HW >> 2 : s.HW;  // items per plane
      const int64_t i1 = (int64_t)(n1 - n0) * per;
      for (int64_t i = threadIdx.x; i < i1; i += kThreads) {
        const int n = n0 + (int)(i / per), r = (int)(i % per);
        const int64_t base = ((int64_t)n * s.C + c) * s.HW;
        f(base + (VEC ? 4 * r : r));
      }
      return;
    }
  }
  for (int n = n0; n < n1; ++n) {
    const int64_t base = ((int64_t)n * s.C + c) * s.HW;
    if constexpr (VEC) {
      const int q0 = r0 >> 2, q1 = r1 >> 2;   // float4 range
      int q = q0 + threadIdx.x;
      for (; q + 3 * kThreads < q1; q += 4 * kThreads) {
#pragma unroll
        for (int u = 0; u < 4; ++u) f(base + 4 * (int64_t)(q + u * kThreads));
      }
      for (; q < q1; q += kThreads) f(base + 4 * (int64_t)q);
    } else {
      int e = r0 + threadIdx.x;
      for (; e + 3 * kThreads < r1; e += 4 * kThreads) {
#pragma unroll
        for (int u = 0; u < 4; ++u) f(base + e + u * kThreads);
      }
      for (; e < r1; e += kThreads) f(base + e);
    }
  }
}

typedef float nf4 __attribute__((ext_vector_type(4)));
// streaming (non-temporal) 16-byte load: the data is touched once per pass
__device__ __forceinline__ float4 ld4(const float* p) {
  const nf4 v = __builtin_nontemporal_load(reinterpret_cast<const nf4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// Pass 1: per-segment sums of g and g*x_norm.  ACT and BN are compile-time so the
// streaming loop has no branches around its loads.  With fixed statistics dz does
// not depend on the sums, so this pass also writes dz = gamma/sqrt(var+eps) * g
// and is the only streaming pass.
template <bool VEC, int ACT, int BN>
__global__ __launch_bounds__(kThreads) void actbn_reduce(
    SegGeom s, const float* delta, const float* __restrict__ y, const float* __restrict__ xn,
    float slope, int act_rt, const float* __restrict__ var, const float* __restrict__ gamma,
    float eps, float* dz /* no batch statistics only, NULL: not written; may alias delta */,
    float2* __restrict__ part) {
  const int c = blockIdx.x / s.nseg, sg = blockIdx.x % s.nseg;
  float sg_ = 0.f, sgx = 0.f;
  const int act = ACT == kActAny ? act_rt : ACT;
  constexpr bool has_y = ACT != CBB_ACT_LINEAR, has_x = BN != kBnNone, fixed = BN == kBnFixed;
  // dz does not depend on the sums without batch statistics: written in this pass
  constexpr bool one_pass = BN != kBnBatch;
  const float ka = fixed ? gamma[c] / sqrtf(var[c] + eps) : 1.f;
  if constexpr (VEC) {
    for_segment<true>(s, c, sg, [&](int64_t o) {
      float4 d = ld4(delta + o);
      if (has_y) {
        const float4 yy = ld4(y + o);
        d.x *= act_grad(act, slope, yy.x);
        d.y *= act_grad(act, slope, yy.y);
        d.z *= act_grad(act, slope, yy.z);
        d.w *= act_grad(act, slope, yy.w);
      }
      sg_ += (d.x + d.y) + (d.z + d.w);
      if (has_x) {
        const float4 x = ld4(xn + o);
        sgx += (d.x * x.x + d.y * x.y) + (d.z * x.z + d.w * x.w);
      }
      if (one_pass && dz)
        *reinterpret_cast<float4*>(dz + o) = make_float4(ka * d.x, ka * d.y, ka * d.z, ka * d.w);
    });
  } else {
    for_segment<false>(s, c, sg, [&](int64_t o) {
      float d = delta[o];
      if (has_y) d *= act_grad(act, slope, y[o]);
      sg_ += d;
      if (has_x) sgx += d * xn[o];
      if (one_pass && dz) dz[o] = ka * d;
    });
  }
  __shared__ float red[4];
  sg_ = block_sum_256(sg_, red);
  sgx = block_sum_256(sgx, red);
  if (threadIdx.x == 0) part[(int64_t)c * s.nseg + sg] = make_float2(sg_, sgx);
}

// One pass for a channel that one work-group can hold: the work-group loads the
// whole channel -- TPB threads x NV float4 of g = delta * act'(y) and (BN) of
// x_norm, in registers -- sums g and g*x_norm (fixed tree order), adds the sums
// into dbeta[c] (db without BN) and dgamma[c] (one work-group per channel: no
// other writer), forms the map dz = a*g + b + cc*x_norm (batch statistics; a =
// gamma/sqrt(var+eps), b = cc = 0 with fixed statistics; a = 1 without BN) and
// writes dz -- or, when a gradient kernel forms dz itself, writes the map to
// coef[c], coef[C+c], coef[2C+c] instead.  delta, y and x_norm are read once and
// dz written once: the 16 bytes per element of the touch-once bound, where the
// two-pass form reads the three tensors twice; a bias-only stage is one launch.
// Needs HW % 4 == 0, 16-byte aligned tensors and N*HW/4 <= TPB*NV.
template <int ACT, int BN, int TPB, int NV>
__global__ __launch_bounds__(TPB) void actbn_channel(
    int N, int C, int HW, const float* delta, const float* __restrict__ y,
    const float* __restrict__ xn, float slope, int act_rt, const float* __restrict__ var,
    const float* __restrict__ gamma, float eps, float* dz /* NULL: not written; may alias delta */,
    float* __restrict__ dgamma, float* __restrict__ dbeta_or_db, float* __restrict__ coef) {
  constexpr int NW = TPB / 64;
  const int act = ACT == kActAny ? act_rt : ACT;
  constexpr bool has_y = ACT != CBB_ACT_LINEAR, has_x = BN != kBnNone;
  const int c = blockIdx.x, per = HW >> 2, total = N * per;
  float4 g[NV], x[has_x ? NV : 1];
  int off[NV];   // element offsets (tensors index in int32)
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int e = threadIdx.x + k * TPB;
    const int n = e / per, r = e - n * per;
    off[k] = e < total ? (n * C + c) * HW + 4 * r : -1;
  }
  const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
  // every load of the channel is issued before the first use
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    g[k] = off[k] >= 0 ? ld4(delta + off[k]) : zero;
    if constexpr (has_x) x[k] = off[k] >= 0 ? ld4(xn + off[k]) : zero;
  }
  if constexpr (has_y) {
    float4 yy[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) yy[k] = off[k] >= 0 ? ld4(y + off[k]) : zero;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      g[k].x *= act_grad(act, slope, yy[k].x);
      g[k].y *= act_grad(act, slope, yy[k].y);
      g[k].z *= act_grad(act, slope, yy[k].z);
      g[k].w *= act_grad(act, slope, yy[k].w);
    }
  }
  float sg = 0.f, sgx = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    sg += (g[k].x + g[k].y) + (g[k].z + g[k].w);
    if constexpr (has_x)
      sgx += (g[k].x * x[k].x + g[k].y * x[k].y) + (g[k].z * x[k].z + g[k].w * x[k].w);
  }
  __shared__ float red[2][NW];
  sg = wave_sum(sg);
  if constexpr (has_x) sgx = wave_sum(sgx);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wave] = sg;
    red[1][wave] = sgx;
  }
  __syncthreads();
  sg = 0.f;
  sgx = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    sg += red[0][w];
    sgx += red[1][w];
  }
  float ka = 1.f, kb = 0.f, kc = 0.f;
  if constexpr (has_x) ka = gamma[c] / sqrtf(var[c] + eps);
  if constexpr (BN == kBnBatch) {
    const float inv_m = 1.f / (float)((int64_t)N * HW);
    kb = -ka * (sg * inv_m);
    kc = -ka * (sgx * inv_m);
  }
  if (threadIdx.x == 0) {
    dbeta_or_db[c] += sg;
    if constexpr (has_x) dgamma[c] += sgx;
    if (coef) {
      coef[c] = ka;
      coef[C + c] = kb;
      coef[2 * C + c] = kc;
    }
  }
  if (coef || !dz) return;
#pragma unroll
  for (int k = 0; k < NV; ++k)
    if (off[k] >= 0) {
      float4 v;
      if constexpr (has_x)
        v = make_float4(ka * g[k].x + kb + kc * x[k].x, ka * g[k].y + kb + kc * x[k].y,
                        ka * g[k].z + kb + kc * x[k].z, ka * g[k].w + kb + kc * x[k].w);
      else
        v = g[k];
      *reinterpret_cast<float4*>(dz + off[k]) = v;
    }
}

// Fold the nseg partials of channel c in a fixed order; every thread gets the sums.
__device__ __forceinline__ float2 fold_partials(const float2* __restrict__ part, int c, int nseg,
                                                float* red) {
  float a = 0.f, b = 0.f;
  for (int k = threadIdx.x; k < nseg; k += kThreads) {
    const float2 v = part[(int64_t)c * nseg + k];
    a += v.x;
    b += v.y;
  }
  a = block_sum_256(a, red);
  b = block_sum_256(b, red);
  return make_float2(a, b);
}

// bn = 1: dz = a*g + b + cc*x_norm with a = gamma/sqrt(var+eps), b = -a*mean(g),
//         cc = -a*mean(g*x_norm); dgamma[c] += sum g*x_norm, dbeta[c] += sum g.
// bn = 0: dz = g (only launched when act != LINEAR), db[c] += sum g.
template <bool VEC, int ACT, int BN>
__global__ __launch_bounds__(kThreads) void actbn_apply(
    SegGeom s, const float* delta, const float* __restrict__ y,
    const float* __restrict__ xn, float slope, int act_rt, const float2* __restrict__ part,
    const float* __restrict__ var, const float* __restrict__ gamma, float eps,
    float* dz /* may alias delta */, float* __restrict__ dgamma, float* __restrict__ dbeta_or_db,
    int write_dz) {
  static_assert(BN != kBnFixed, "fixed statistics write dz in pass 1");
  const int act = ACT == kActAny ? act_rt : ACT;
  constexpr bool bn = BN == kBnBatch;
  const int c = blockIdx.x / s.nseg, sg = blockIdx.x % s.nseg;
  __shared__ float red[4];
  const float2 sums = fold_partials(part, c, s.nseg, red);
  if (sg == 0 && threadIdx.x == 0) {
    dbeta_or_db[c] += sums.x;
    if (bn) dgamma[c] += sums.y;
  }
  if (!write_dz) return;
  float ka = 1.f, kb = 0.f, kc = 0.f;
  if (bn) {
    const float inv_m = 1.f / (float)s.M;
    ka = gamma[c] / sqrtf(var[c] + eps);
    kb = -ka * (sums.x * inv_m);
    kc = -ka * (sums.y * inv_m);
  }
  constexpr bool has_y = ACT != CBB_ACT_LINEAR;
  if constexpr (VEC) {
    for_segment<true>(s, c, sg, [&](int64_t o) {
      float4 d = ld4(delta + o);
      if (has_y) {
        const float4 yy = ld4(y + o);
        d.x *= act_grad(act, slope, yy.x);
        d.y *= act_grad(act, slope, yy.y);
        d.z *= act_grad(act, slope, yy.z);
        d.w *= act_grad(act, slope, yy.w);
      }
      if (bn) {
        const float4 x = ld4(xn + o);
        d.x = ka * d.x + kb + kc * x.x;
        d.y = ka * d.y + kb + kc * x.y;
        d.z = ka * d.z + kb + kc * x.z;
        d.w = ka * d.w + kb + kc * x.w;
      }
      *reinterpret_cast<float4*>(dz + o) = d;
    });
  } else {
    for_segment<false>(s, c, sg, [&](int64_t o) {
      float d = delta[o];
      if (has_y) d *= act_grad(act, slope, y[o]);
      if (bn) d = ka * d + kb + kc * xn[o];
      dz[o] = d;
    });
  }
}

// Fixed statistics, pass 2: one work-group per channel adds the channel's sums,
// folded in a fixed order, into dgamma / dbeta.
__global__ __launch_bounds__(kThreads) void actbn_fold(const float2* __restrict__ part, int nseg,
                                                       float* __restrict__ dgamma,
                                                       float* __restrict__ dbeta) {
  __shared__ float red[4];
  const int c = blockIdx.x;
  const float2 sums = fold_partials(part, c, nseg, red);
  if (threadIdx.x == 0) {
    dbeta[c] += sums.x;
    if (dgamma) dgamma[c] += sums.y;
  }
}

// sums[c] = the channel's partials folded in the fixed order of actbn_apply.
__global__ __launch_bounds__(kThreads) void bn_sums_fold(const float2* __restrict__ part, int nseg,
                                                         float2* __restrict__ sums) {
  __shared__ float red[4];
  const int c = blockIdx.x;
  const float2 v = fold_partials(part, c, nseg, red);
  if (threadIdx.x == 0) sums[c] = v;
}

// Given sums as partials of nseg segments: segment 0 holds the sum, the rest zero.
__global__ __launch_bounds__(kThreads) void bn_sums_expand(const float2* __restrict__ sums,
                                                           float2* __restrict__ part, int nseg) {
  const int c = blockIdx.x;
  for (int j = threadIdx.x; j < nseg; j += kThreads)
    part[(int64_t)c * nseg + j] = j == 0 ? sums[c] : make_float2(0.f, 0.f);
}

// Pass 2 when dz is formed later by its consumer: one work-group per channel
// folds the sums (the order actbn_apply uses), adds them into dgamma / dbeta (or
// db) and writes the channel's map dz = a*g + b + cc*x_norm as coef[c], coef[C+c],
// coef[2C+c] (no BN: a = 1; fixed statistics: b = cc = 0).
__global__ __launch_bounds__(kThreads) void actbn_coef(const float2* __restrict__ part, int nseg,
                                                       int64_t M, int C, int bn,
                                                       const float* __restrict__ var,
                                                       const float* __restrict__ gamma, float eps,
                                                       float* __restrict__ dgamma,
                                                       float* __restrict__ dbeta_or_db,
                                                       float* __restrict__ coef) {
  __shared__ float red[4];
  const int c = blockIdx.x;
  const float2 sums = fold_partials(part, c, nseg, red);
  if (threadIdx.x != 0) return;
  dbeta_or_db[c] += sums.x;
  float ka = 1.f, kb = 0.f, kc = 0.f;
  if (bn != kBnNone) {
    dgamma[c] += sums.y;
    ka = gamma[c] / sqrtf(var[c] + eps);
    if (bn == kBnBatch) {
      const float inv_m = 1.f / (float)M;
      kb = -ka * (sums.x * inv_m);
      kc = -ka * (sums.y * inv_m);
    }
  }
  coef[c] = ka;
  coef[C + c] = kb;
  coef[2 * C + c] = kc;
}

__global__ __launch_bounds__(kThreads) void act_backward_kernel(int act, float slope,
                                                                const float* __restrict__ y,
                                                                const float* delta,
                                                                float* g /* may alias delta */,
                                                                int64_t count) {
  const int64_t n4 = count >> 2;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    float4 d = reinterpret_cast<const float4*>(delta)[i];
    const float4 yy = reinterpret_cast<const float4*>(y)[i];
    d.x *= act_grad(act, slope, yy.x);
    d.y *= act_grad(act, slope, yy.y);
    d.z *= act_grad(act, slope, yy.z);
    d.w *= act_grad(act, slope, yy.w);
    reinterpret_cast<float4*>(g)[i] = d;
  }
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += stride)
    g[i] = delta[i] * act_grad(act, slope, y[i]);
}

__global__ __launch_bounds__(kThreads) void act_backward_scalar(int act, float slope,
                                                                const float* __restrict__ y,
                                                                const float* delta,
                                                                float* g /* may alias delta */,
                                                                int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += stride)
    g[i] = delta[i] * act_grad(act, slope, y[i]);
}

// ---------------------------------------------------------------------------
// Forward of the block after the convolution (the tensors the backward reads):
// batch statistics of z per channel over (batch, space) -- the mean, then the
// biased variance E[(z - mean)^2] ("Understanding BatchNorm", Forward_cpu; the
// YOLOv3 page's mean_cpu / variance_cpu) -- x_norm = (z - mean)/sqrt(var + eps),
// u = gamma x_norm + beta (scale_bias, add_bias), y = act(u) (section 7's
// *_activate functions).
// ---------------------------------------------------------------------------

// Batch statistics in one pass.  Each thread sums d = z - K and d^2 with K its own
// first element (a shift inside the data keeps the sums small), turns them into
// (count, mean, M2 = sum of squared deviations), and the work-group merges the 256
// triples pairwise in a fixed tree (merge_moments) into its segment's (mean, M2);
// bnf_stats_fold merges the segments in order.

// elements in segment sg of a channel (the split of for_segment)
__device__ __forceinline__ int64_t seg_count(const SegGeom& s, int sg) {
  if (s.parts > 1) {
    const int part = sg % s.parts, r0 = part * s.chunk;
    return min(s.HW, r0 + s.chunk) - r0;
  }
  const int n0 = sg * s.group, n1 = min(s.N, n0 + s.group);
  return (int64_t)(n1 - n0) * s.HW;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void bnf_stats(SegGeom s, const float* __restrict__ z,
                                                      float2* __restrict__ part) {
  const int c = blockIdx.x / s.nseg, sg = blockIdx.x % s.nseg;
  float k = 0.f, s1 = 0.f, s2 = 0.f;
  int cnt = 0;
  auto add = [&](float v) {
    if (cnt == 0) k = v;
    const float d = v - k;
    s1 += d;
    s2 += d * d;
    ++cnt;
  };
  if constexpr (VEC) {
    for_segment<true>(s, c, sg, [&](int64_t o) {
      const float4 v = ld4(z + o);
      add(v.x);
      add(v.y);
      add(v.z);
      add(v.w);
    });
  } else {
    for_segment<false>(s, c, sg, [&](int64_t o) { add(z[o]); });
  }
  __shared__ Moments red[kThreads];
  Moments m{0.f, 0.f, 0.f};
  if (cnt > 0) {
    const float n = (float)cnt, mu = s1 / n;
    m = Moments{n, k + mu, fmaxf(s2 - s1 * mu, 0.f)};
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int stride = kThreads / 2; stride > 0; stride >>= 1) {
    if ((int)threadIdx.x < stride) red[threadIdx.x] = merge_moments(red[threadIdx.x], red[threadIdx.x + stride]);
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = make_float2(red[0].mean, red[0].m2);
}

// mean[c], var[c] (biased) from the channel's segments, merged in order in double.
__global__ __launch_bounds__(64) void bnf_stats_fold(SegGeom s, const float2* __restrict__ part,
                                                     float* __restrict__ mean,
                                                     float* __restrict__ var) {
  const int c = blockIdx.x;
  if (threadIdx.x != 0) return;
  double n = 0.0, mu = 0.0, m2 = 0.0;
  for (int sg = 0; sg < s.nseg; ++sg) {
    const double nb = (double)seg_count(s, sg);
    const float2 v = part[(int64_t)c * s.nseg + sg];
    const double tot = n + nb, d = (double)v.x - mu;
    mu += d * nb / tot;
    m2 += (double)v.y + d * d * n * nb / tot;
    n = tot;
  }
  mean[c] = (float)mu;
  var[c] = (float)(m2 / n);
}


// BN: xn holds z on entry and x_norm on exit; y = act(gamma x_norm + beta).
// No BN: y holds z (+ bias) on entry and act of it on exit (xn == y).
template <bool VEC, bool BN>
__global__ __launch_bounds__(kThreads) void bnf_apply(SegGeom s, float* xn, float* y,
                                                      const float* __restrict__ mean,
                                                      const float* __restrict__ var,
                                                      const float* __restrict__ gamma,
                                                      const float* __restrict__ beta, float eps,
                                                      int act, float slope) {
  const int c = blockIdx.x / s.nseg, sg = blockIdx.x % s.nseg;
  float mu = 0.f, inv = 1.f, ga = 1.f, be = 0.f;
  if (BN) {
    mu = mean[c];
    inv = 1.f / sqrtf(var[c] + eps);
    ga = gamma[c];
    be = beta[c];
  }
  auto one = [&](float v, float* xo) {
    float u = v;
    if (BN) {
      const float xh = (v - mu) * inv;
      *xo = xh;
      u = ga * xh + be;
    }
    return act_fwd(act, slope, u);
  };
  if constexpr (VEC) {
    for_segment<true>(s, c, sg, [&](int64_t o) {
      const float4 v = *reinterpret_cast<const float4*>(xn + o);
      float4 xh = v, r;
      r.x = one(v.x, &xh.x);
      r.y = one(v.y, &xh.y);
      r.z = one(v.z, &xh.z);
      r.w = one(v.w, &xh.w);
      if (BN) *reinterpret_cast<float4*>(xn + o) = xh;
      *reinterpret_cast<float4*>(y + o) = r;
    });
  } else {
    for_segment<false>(s, c, sg, [&](int64_t o) {
      float xh = 0.f;
      const float r = one(xn[o], &xh);
      if (BN) xn[o] = xh;
      y[o] = r;
    });
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
SegGeom plan_seg(int N, int C, int64_t HW) {
  SegGeom s;
  s.N = N;
  s.C = C;
  s.HW = (int)HW;
  s.M = (int64_t)N * HW;
  // ~1024 work-groups in total (measured best on MI355X for these streaming passes),
  // each streaming at least ~4096 elements
  const int64_t target = std::max<int64_t>(1, std::min<int64_t>(ceil_div(1024, C), s.M / 4096));
  if (HW >= kPlaneSplit) {
    int64_t parts = std::max<int64_t>(1, ceil_div(target, N));
    int64_t chunk = ceil_div(ceil_div(HW, parts), 4) * 4;
    s.parts = (int)ceil_div(HW, chunk);
    s.chunk = (int)chunk;
    s.group = 1;
    s.nseg = N * s.parts;
  } else {
    s.parts = 1;
    s.chunk = (int)HW;
    s.group = (int)std::max<int64_t>(1, ceil_div(N, target));
    s.nseg = (int)ceil_div(N, s.group);
  }
  return s;
}

size_t actbn_workspace(int N, int C, int64_t HW) {
  const SegGeom s = plan_seg(N, C, HW);
  return (size_t)C * s.nseg * sizeof(float2);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// float4 per thread of the one-pass form: channels of up to 256 x 6 x 4 = 6144
// elements take 256-thread work-groups, up to 1024 x 6 x 4 = 24576 elements (BN) or
// 1024 x 10 x 4 = 40960 (no BN: no x_norm held) 1024.
constexpr int kChanNV = 6, kChanNV1024 = 10;

// g/BN stage of a conv block, or a standalone BN backward (act = LINEAR).
// Writes dz (when needed), adds to dgamma/dbeta (BN) or db (no BN).
template <bool VEC, int ACT, int BN>
static void launch_actbn_t(const SegGeom& s, unsigned blocks, int act, const float* delta,
                           const float* y, const float* xn, float slope, const float* var,
                           const float* gamma, float eps, float* dz, float* dgamma,
                           float* dbeta_or_db, float2* part, int write_dz, float* coef,
                           const float2* sums, hipStream_t st) {
  const float* xr = BN != kBnNone ? xn : nullptr;
  if (sums) {
    // batch statistics whose sums another call produced: no reduction pass
    if constexpr (BN == kBnBatch) {
      if (coef) {
        actbn_coef<<<(unsigned)s.C, kThreads, 0, st>>>(sums, 1, s.M, s.C, BN, var, gamma, eps,
                                                      dgamma, dbeta_or_db, coef);
        note_launch("actbn_coef", st);
        return;
      }
      bn_sums_expand<<<(unsigned)s.C, kThreads, 0, st>>>(sums, part, s.nseg);
      note_launch("bn_sums_expand", st);
      actbn_apply<VEC, ACT, BN><<<blocks, kThreads, 0, st>>>(s, delta, y, xn, slope, act, part,
                                                             var, gamma, eps, dz, dgamma,
                                                             dbeta_or_db, write_dz);
      note_launch("actbn_apply", st);
    }
    return;
  }
  // A channel that one work-group holds in registers takes one pass for any mode:
  // sums, then dz (or the map for a kernel that forms dz itself).
  const int64_t q = (int64_t)s.N * s.HW / 4;
  if (VEC && q <= 256 * kChanNV) {
    actbn_channel<ACT, BN, 256, kChanNV><<<(unsigned)s.C, 256, 0, st>>>(
        s.N, s.C, s.HW, delta, y, xr, slope, act, var, gamma, eps, write_dz ? dz : nullptr,
        dgamma, dbeta_or_db, coef);
    note_launch("actbn_channel", st);
    return;
  }
  constexpr int NV1024 = BN != kBnNone ? kChanNV : kChanNV1024;   // g and x_norm: 128 VGPRs
  if (VEC && q <= 1024 * NV1024) {
    actbn_channel<ACT, BN, 1024, NV1024><<<(unsigned)s.C, 1024, 0, st>>>(
        s.N, s.C, s.HW, delta, y, xr, slope, act, var, gamma, eps, write_dz ? dz : nullptr,
        dgamma, dbeta_or_db, coef);
    note_launch("actbn_channel", st);
    return;
  }
  if (coef || BN != kBnBatch) {
    // one streaming pass (dz written in it, or formed later from coef)
    actbn_reduce<VEC, ACT, BN><<<blocks, kThreads, 0, st>>>(
        s, delta, y, xr, slope, act, var, gamma, eps, coef || !write_dz ? nullptr : dz, part);
    note_launch("actbn_reduce", st);
    if (coef) {
      actbn_coef<<<(unsigned)s.C, kThreads, 0, st>>>(part, s.nseg, s.M, s.C, BN, var, gamma,
                                                    eps, dgamma, dbeta_or_db, coef);
      note_launch("actbn_coef", st);
    } else {
      actbn_fold<<<(unsigned)s.C, kThreads, 0, st>>>(part, s.nseg,
                                                    BN == kBnNone ? nullptr : dgamma,
                                                    dbeta_or_db);
      note_launch("actbn_fold", st);
    }
    return;
  }
  // batch statistics on a channel too large for one work-group: dz needs the
  // channel's sums, so the data is streamed twice
  if constexpr (BN == kBnBatch) {
    actbn_reduce<VEC, ACT, BN><<<blocks, kThreads, 0, st>>>(s, delta, y, xr, slope, act, var,
                                                            gamma, eps, nullptr, part);
    note_launch("actbn_reduce", st);
    actbn_apply<VEC, ACT, BN><<<blocks, kThreads, 0, st>>>(s, delta, y, xn, slope, act, part, var,
                                                           gamma, eps, dz, dgamma, dbeta_or_db,
                                                           write_dz);
    note_launch("actbn_apply", st);
  }
}

template <bool VEC, int ACT>
static void launch_actbn_a(const SegGeom& s, unsigned blocks, int act, int bn, const float* delta,
                           const float* y, const float* xn, float slope, const float* var,
                           const float* gamma, float eps, float* dz, float* dgamma,
                           float* dbeta_or_db, float2* part, int write_dz, float* coef,
                           const float2* sums, hipStream_t st) {
#define CBB_ACTBN(B)                                                                        \
  launch_actbn_t<VEC, ACT, B>(s, blocks, act, delta, y, xn, slope, var, gamma, eps, dz, dgamma, \
                              dbeta_or_db, part, write_dz, coef, sums, st)
  if (bn == kBnFixed)
    CBB_ACTBN(kBnFixed);
  else if (bn == kBnBatch)
    CBB_ACTBN(kBnBatch);
  else
    CBB_ACTBN(kBnNone);
#undef CBB_ACTBN
}

template <bool VEC>
static void launch_actbn_v(const SegGeom& s, unsigned blocks, int act, int bn, const float* delta,
                           const float* y, const float* xn, float slope, const float* var,
                           const float* gamma, float eps, float* dz, float* dgamma,
                           float* dbeta_or_db, float2* part, int write_dz, float* coef,
                           const float2* sums, hipStream_t st) {
#define CBB_ACTBN(A)                                                                          \
  launch_actbn_a<VEC, A>(s, blocks, act, bn, delta, y, xn, slope, var, gamma, eps, dz, dgamma, \
                         dbeta_or_db, part, write_dz, coef, sums, st)
  switch (act) {
    case CBB_ACT_LINEAR: CBB_ACTBN(CBB_ACT_LINEAR); break;
    case CBB_ACT_LEAKY: CBB_ACTBN(CBB_ACT_LEAKY); break;
    case CBB_ACT_LOGISTIC: CBB_ACTBN(CBB_ACT_LOGISTIC); break;
    case CBB_ACT_RELU: CBB_ACTBN(CBB_ACT_RELU); break;
    default: CBB_ACTBN(kActAny); break;
  }
#undef CBB_ACTBN
}

// g/BN stage of a conv block, or a standalone BN backward (act = LINEAR).
// bn: 0 none (db += sum g), 1 batch statistics, 2 fixed statistics.  coef != NULL:
// dz is not written; the per-channel map that forms it goes to coef[3C] instead.
int launch_actbn(int N, int C, int64_t HW, const float* delta, const float* y, const float* xn,
                 int act, float slope, const float* var, const float* gamma, float eps, int bn,
                 float* dz, float* dgamma, float* dbeta_or_db, void* ws, hipStream_t st,
                 float* coef, const float2* sums) {
  const SegGeom s = plan_seg(N, C, HW);
  float2* part = reinterpret_cast<float2*>(ws);
  const bool vec = (HW % 4 == 0) && aligned16(delta) && (!y || aligned16(y)) &&
                   (!xn || aligned16(xn)) && (!dz || aligned16(dz));
  const unsigned blocks = (unsigned)((int64_t)C * s.nseg);
  const int write_dz = bn || act != CBB_ACT_LINEAR;
  if (sums && bn != kBnBatch) return CBB_EINVAL;
  if (vec)
    launch_actbn_v<true>(s, blocks, act, bn, delta, y, xn, slope, var, gamma, eps, dz, dgamma,
                         dbeta_or_db, part, write_dz, coef, sums, st);
  else
    launch_actbn_v<false>(s, blocks, act, bn, delta, y, xn, slope, var, gamma, eps, dz, dgamma,
                          dbeta_or_db, part, write_dz, coef, sums, st);
  return check_error("actbn_reduce/actbn_apply");
}

size_t bn_sums_workspace(int N, int C, int64_t HW) { return actbn_workspace(N, C, HW); }

template <bool VEC, int ACT>
static void launch_bn_sums_t(const SegGeom& s, unsigned blocks, int act, const float* delta,
                             const float* y, const float* xn, float slope, float2* part,
                             hipStream_t st) {
  actbn_reduce<VEC, ACT, kBnBatch><<<blocks, kThreads, 0, st>>>(s, delta, y, xn, slope, act,
                                                                nullptr, nullptr, 0.f, nullptr,
                                                                part);
  note_launch("actbn_reduce", st);
}

int launch_bn_sums(int N, int C, int64_t HW, const float* delta, const float* y, const float* xn,
                   int act, float slope, void* ws, float2* sums, hipStream_t st) {
  const SegGeom s = plan_seg(N, C, HW);
  float2* part = reinterpret_cast<float2*>(ws);
  const bool vec = (HW % 4 == 0) && aligned16(delta) && (!y || aligned16(y)) && aligned16(xn);
  const unsigned blocks = (unsigned)((int64_t)C * s.nseg);
#define CBB_SUMS(V, A) launch_bn_sums_t<V, A>(s, blocks, act, delta, y, xn, slope, part, st)
  if (vec) {
    if (act == CBB_ACT_LEAKY) CBB_SUMS(true, CBB_ACT_LEAKY);
    else if (act == CBB_ACT_LINEAR) CBB_SUMS(true, CBB_ACT_LINEAR);
    else CBB_SUMS(true, kActAny);
  } else {
    if (act == CBB_ACT_LEAKY) CBB_SUMS(false, CBB_ACT_LEAKY);
    else if (act == CBB_ACT_LINEAR) CBB_SUMS(false, CBB_ACT_LINEAR);
    else CBB_SUMS(false, kActAny);
  }
#undef CBB_SUMS
  return launch_bn_sums_fold(part, C, s.nseg, sums, st);
}

int launch_bn_sums_fold(const float2* part, int C, int nseg, float2* sums, hipStream_t st) {
  bn_sums_fold<<<(unsigned)C, kThreads, 0, st>>>(part, nseg, sums);
  note_launch("bn_sums_fold", st);
  return check_error("bn_sums_fold");
}

// Forward after the convolution (see bnf_apply).  bn: 0 none (z + bias already in y),
// 1 batch statistics (written to mean / var), 2 fixed statistics (read).
int launch_bn_act_forward(int N, int C, int64_t HW, int bn, float eps, int act, float slope,
                          const float* gamma, const float* beta, float* mean, float* var,
                          float* xn, float* y, void* ws, hipStream_t st) {
  const SegGeom s = plan_seg(N, C, HW);
  const unsigned blocks = (unsigned)((int64_t)C * s.nseg);
  const bool vec = (HW % 4 == 0) && aligned16(xn) && aligned16(y);
  if (bn == 1) {
    // one reading pass: per-segment (mean, M2), merged per channel
    float2* mp = reinterpret_cast<float2*>(ws);
    if (vec)
      bnf_stats<true><<<blocks, kThreads, 0, st>>>(s, xn, mp);
    else
      bnf_stats<false><<<blocks, kThreads, 0, st>>>(s, xn, mp);
    note_launch("bnf_stats", st);
    bnf_stats_fold<<<(unsigned)C, 64, 0, st>>>(s, mp, mean, var);
    note_launch("bnf_stats_fold", st);
  }
  if (bn) {
    if (vec)
      bnf_apply<true, true><<<blocks, kThreads, 0, st>>>(s, xn, y, mean, var, gamma, beta, eps,
                                                          act, slope);
    else
      bnf_apply<false, true><<<blocks, kThreads, 0, st>>>(s, xn, y, mean, var, gamma, beta, eps,
                                                           act, slope);
  } else if (act != CBB_ACT_LINEAR) {
    if (vec)
      bnf_apply<true, false><<<blocks, kThreads, 0, st>>>(s, y, y, nullptr, nullptr, nullptr,
                                                           nullptr, eps, act, slope);
    else
      bnf_apply<false, false><<<blocks, kThreads, 0, st>>>(s, y, y, nullptr, nullptr, nullptr,
                                                            nullptr, eps, act, slope);
  }
  if (bn || act != CBB_ACT_LINEAR) note_launch("bnf_apply", st);
  return check_error("bnf_stats/bnf_stats_fold/bnf_apply");
}

int launch_act_backward(int act, float slope, const float* y, const float* delta, float* g,
                        int64_t count, hipStream_t st) {
  if (aligned16(y) && aligned16(delta) && aligned16(g)) {
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(ceil_div(count, 4 * kThreads), 8192));
    act_backward_kernel<<<(unsigned)blocks, kThreads, 0, st>>>(act, slope, y, delta, g, count);
  } else {
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(ceil_div(count, kThreads), 8192));
    act_backward_scalar<<<(unsigned)blocks, kThreads, 0, st>>>(act, slope, y, delta, g, count);
  }
  return check_launch("act_backward_kernel", st);
}

}  // namespace cbb
