// bn_act.hip -- activation gradient + batch-norm backward (or bias sum) as two
// streaming passes over the conv output, bandwidth-bound by design.
//
// "YOLOv3 backpropagation: full-flow source analysis" (suzhouguqin.com):
//   section 3.1 gradient_array: g = delta * act'(y), act' read from the output;
//   section 4 backward_batchnorm_layer: dbeta += sum g (backward_bias),
//   dgamma += sum g*x_norm (backward_scale_cpu), then the input gradient;
//   section 7: leaky (y>0 ? 1 : .1), logistic (1-y)y, linear 1, relu (y>0).
// "Understanding BatchNorm" (javaforall.cn): Caffe's closed form
//   dz = (g' - mean(g') - mean(g' x_norm) x_norm) / sqrt(var + eps), g' = gamma g.
//
// Pass 1 (actbn_reduce) : each work-group sums (g, g*x_norm) over one segment
//                         of one channel -> workspace partials[c][seg].
// Pass 2 (actbn_apply)  : each work-group first folds its channel's partials in
//                         a fixed order (deterministic), derives the per-channel
//                         affine map dz = a*g + b + c*x_norm, writes dz for its
//                         segment; segment 0 also adds the channel's sums into
//                         dgamma / dbeta (or db).
// A channel's data is N planes of HW floats, (n*C + c)*HW apart; a segment is a
// contiguous run of the flattened (n, hw) index.
#include "cbb_internal.h"

namespace cbb {

__device__ __forceinline__ float act_grad(int act, float slope, float y) {
  switch (act) {
    case CBB_ACT_LEAKY: return y > 0.f ? 1.f : slope;
    case CBB_ACT_LOGISTIC: return (1.f - y) * y;
    case CBB_ACT_RELU: return y > 0.f ? 1.f : 0.f;
    default: return 1.f;
  }
}

struct SegGeom {
  int N, C, HW;
  int64_t M;      // N*HW elements per channel
  int nseg;       // segments per channel
  int64_t seg;    // elements per segment (multiple of 4 when VEC)
};

// Visit the elements of segment `sg` of channel `c`: f(offset) for scalar
// offsets, in float4 groups when VEC (HW % 4 == 0, so a group never crosses a
// plane).  Thread t takes groups t, t+256, ... of the segment.
template <bool VEC, class F>
__device__ __forceinline__ void for_segment(const SegGeom& s, int c, int sg, F&& f) {
  const int64_t e0 = (int64_t)sg * s.seg;
  const int64_t e1 = min(s.M, e0 + s.seg);
  if constexpr (VEC) {
    const int HW4 = s.HW >> 2;
    int64_t g = (e0 >> 2) + threadIdx.x;
    const int64_t gend = e1 >> 2;
    if (g >= gend) return;
    int n = (int)(g / HW4);
    int i4 = (int)(g - (int64_t)n * HW4);
    for (; g < gend; g += kThreads) {
      f(((int64_t)n * s.C + c) * s.HW + 4 * i4);
      i4 += kThreads;
      while (i4 >= HW4) {
        i4 -= HW4;
        ++n;
      }
    }
  } else {
    int64_t e = e0 + threadIdx.x;
    if (e >= e1) return;
    int n = (int)(e / s.HW);
    int i = (int)(e - (int64_t)n * s.HW);
    for (; e < e1; e += kThreads) {
      f(((int64_t)n * s.C + c) * s.HW + i);
      i += kThreads;
      while (i >= s.HW) {
        i -= s.HW;
        ++n;
      }
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void actbn_reduce(SegGeom s, const float* __restrict__ delta,
                                                         const float* __restrict__ y,
                                                         const float* __restrict__ xn, int act,
                                                         float slope, float2* __restrict__ part) {
  const int c = blockIdx.x / s.nseg, sg = blockIdx.x % s.nseg;
  float sg_ = 0.f, sgx = 0.f;
  const bool has_y = act != CBB_ACT_LINEAR, has_x = xn != nullptr;
  if constexpr (VEC) {
    for_segment<true>(s, c, sg, [&](int64_t o) {
      float4 d = *reinterpret_cast<const float4*>(delta + o);
      if (has_y) {
        const float4 yy = *reinterpret_cast<const float4*>(y + o);
        d.x *= act_grad(act, slope, yy.x);
        d.y *= act_grad(act, slope, yy.y);
        d.z *= act_grad(act, slope, yy.z);
        d.w *= act_grad(act, slope, yy.w);
      }
      sg_ += (d.x + d.y) + (d.z + d.w);
      if (has_x) {
        const float4 x = *reinterpret_cast<const float4*>(xn + o);
        sgx += (d.x * x.x + d.y * x.y) + (d.z * x.z + d.w * x.w);
      }
    });
  } else {
    for_segment<false>(s, c, sg, [&](int64_t o) {
      float d = delta[o];
      if (has_y) d *= act_grad(act, slope, y[o]);
      sg_ += d;
      if (has_x) sgx += d * xn[o];
    });
  }
  __shared__ float red[4];
  sg_ = block_sum_256(sg_, red);
  sgx = block_sum_256(sgx, red);
  if (threadIdx.x == 0) part[blockIdx.x] = make_float2(sg_, sgx);
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
template <bool VEC>
__global__ __launch_bounds__(kThreads) void actbn_apply(
    SegGeom s, const float* delta, const float* __restrict__ y,
    const float* __restrict__ xn, int act, float slope, const float2* __restrict__ part,
    const float* __restrict__ var, const float* __restrict__ gamma, float eps, int bn,
    float* dz /* may alias delta */, float* __restrict__ dgamma, float* __restrict__ dbeta_or_db,
    int write_dz) {
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
  const bool has_y = act != CBB_ACT_LINEAR;
  if constexpr (VEC) {
    for_segment<true>(s, c, sg, [&](int64_t o) {
      float4 d = *reinterpret_cast<const float4*>(delta + o);
      if (has_y) {
        const float4 yy = *reinterpret_cast<const float4*>(y + o);
        d.x *= act_grad(act, slope, yy.x);
        d.y *= act_grad(act, slope, yy.y);
        d.z *= act_grad(act, slope, yy.z);
        d.w *= act_grad(act, slope, yy.w);
      }
      if (bn) {
        const float4 x = *reinterpret_cast<const float4*>(xn + o);
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
// Host side.
// ---------------------------------------------------------------------------
SegGeom plan_seg(int N, int C, int64_t HW) {
  SegGeom s;
  s.N = N;
  s.C = C;
  s.HW = (int)HW;
  s.M = (int64_t)N * HW;
  // ~2048 work-groups in total, each streaming at least 4096 elements.
  int64_t nseg = ceil_div(2048, C);
  nseg = std::min<int64_t>(nseg, std::max<int64_t>(1, s.M / 4096));
  nseg = std::max<int64_t>(1, nseg);
  int64_t seg = ceil_div(s.M, nseg);
  seg = ceil_div(seg, 4) * 4;
  s.seg = seg;
  s.nseg = (int)ceil_div(s.M, seg);
  return s;
}

size_t actbn_workspace(int N, int C, int64_t HW) {
  const SegGeom s = plan_seg(N, C, HW);
  return (size_t)C * s.nseg * sizeof(float2);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// g/BN stage of a conv block, or a standalone BN backward (act = LINEAR).
// Writes dz (when needed), adds to dgamma/dbeta (bn) or db (!bn).
int launch_actbn(int N, int C, int64_t HW, const float* delta, const float* y, const float* xn,
                 int act, float slope, const float* var, const float* gamma, float eps, int bn,
                 float* dz, float* dgamma, float* dbeta_or_db, void* ws, hipStream_t st) {
  const SegGeom s = plan_seg(N, C, HW);
  float2* part = reinterpret_cast<float2*>(ws);
  const bool vec = (HW % 4 == 0) && aligned16(delta) && (!y || aligned16(y)) &&
                   (!xn || aligned16(xn)) && (!dz || aligned16(dz));
  const unsigned blocks = (unsigned)((int64_t)C * s.nseg);
  const float* xn_r = bn ? xn : nullptr;
  if (vec)
    actbn_reduce<true><<<blocks, kThreads, 0, st>>>(s, delta, y, xn_r, act, slope, part);
  else
    actbn_reduce<false><<<blocks, kThreads, 0, st>>>(s, delta, y, xn_r, act, slope, part);
  int rc = check_launch("actbn_reduce");
  if (rc) return rc;
  const int write_dz = bn || act != CBB_ACT_LINEAR;
  if (vec)
    actbn_apply<true><<<blocks, kThreads, 0, st>>>(s, delta, y, xn, act, slope, part, var, gamma,
                                                   eps, bn, dz, dgamma, dbeta_or_db, write_dz);
  else
    actbn_apply<false><<<blocks, kThreads, 0, st>>>(s, delta, y, xn, act, slope, part, var, gamma,
                                                    eps, bn, dz, dgamma, dbeta_or_db, write_dz);
  return check_launch("actbn_apply");
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
  return check_launch("act_backward_kernel");
}

}  // namespace cbb
