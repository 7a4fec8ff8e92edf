// depthwise.hip -- gradients of a depthwise convolution (groups = in_c = out_c):
// every channel has its own k x k filter, so there is no contraction over
// channels to put on the matrix cores.  dW is a per-channel streaming reduction
// (like the batch-norm sums) and dX a per-plane stencil; both read x / dz from
// HBM once, neighbouring taps hitting the caches.
//
// Pages: "YOLOv3 backpropagation: full-flow source analysis" (suzhouguqin.com),
// section 3.1 (backward_convolutional_layer per group: with l.groups = l.c the
// gemm of group j is the 1 x (k*k) filter of channel j).  Tap (kh, kw) of output
// (ho, wo) reads input (ho*S + kh*D - P, wo*S + kw*D - P), zero outside.
#include "cbb_internal.h"

namespace cbb {

bool conv_depthwise(const ConvGeom& g) { return g.G > 1 && g.G == g.C && g.G == g.OC; }

// Output positions of a channel (N * OH * OW) are cut into nseg segments.
struct DwiseSeg {
  int nseg;
  int64_t seglen;
};

static DwiseSeg dwise_plan(const ConvGeom& g) {
  const int64_t m = (int64_t)g.N * g.OHW;
  // ~1024 work-groups in total, each over at least ~2048 positions
  const int64_t nseg = std::max<int64_t>(1, std::min<int64_t>(ceil_div(1024, g.C), m / 2048));
  DwiseSeg s;
  s.seglen = ceil_div(m, nseg);
  s.nseg = (int)ceil_div(m, s.seglen);
  return s;
}

// dW partial sums: work-group (c, segment) accumulates all K*K taps of channel c
// over its output positions; part[(c*nseg + seg)*K*K + tap].
template <int K>
__global__ __launch_bounds__(kThreads) void dwise_dw_partial(ConvGeom g, const float* __restrict__ x,
                                                             const float* __restrict__ dz,
                                                             float* __restrict__ part, int nseg,
                                                             int64_t seglen) {
  const int c = blockIdx.x / nseg, sg = blockIdx.x % nseg;
  const int64_t m = (int64_t)g.N * g.OHW;
  const int64_t q0 = (int64_t)sg * seglen, q1 = min(m, q0 + seglen);
  float acc[K * K];
#pragma unroll
  for (int t = 0; t < K * K; ++t) acc[t] = 0.f;
  for (int64_t q = q0 + threadIdx.x; q < q1; q += kThreads) {
    const int n = (int)(q / g.OHW), r = (int)(q - (int64_t)n * g.OHW);
    const int ho = r / g.OW, wo = r - ho * g.OW;
    const float d = dz[((int64_t)n * g.C + c) * g.OHW + r];
    const float* xp = x + ((int64_t)n * g.C + c) * g.HW;
    const int h0 = ho * g.S - g.P, w0 = wo * g.S - g.P;
#pragma unroll
    for (int kh = 0; kh < K; ++kh) {
      const int h = h0 + kh * g.D;
      const bool hv = (unsigned)h < (unsigned)g.H;
#pragma unroll
      for (int kw = 0; kw < K; ++kw) {
        const int w = w0 + kw * g.D;
        if (hv && (unsigned)w < (unsigned)g.W) acc[kh * K + kw] += d * xp[h * g.W + w];
      }
    }
  }
  __shared__ float red[4];
#pragma unroll
  for (int t = 0; t < K * K; ++t) {
    const float v = block_sum_256(acc[t], red);
    if (threadIdx.x == 0) part[((int64_t)c * nseg + sg) * (K * K) + t] = v;
  }
}

// dW[c][tap] += the channel's segment sums, added in segment order.
__global__ __launch_bounds__(64) void dwise_dw_fold(const float* __restrict__ part, int nseg,
                                                    int kk, float* __restrict__ dw) {
  const int c = blockIdx.x, t = threadIdx.x;
  if (t >= kk) return;
  float s = 0.f;
  for (int sg = 0; sg < nseg; ++sg) s += part[((int64_t)c * nseg + sg) * kk + t];
  dw[(int64_t)c * kk + t] += s;
}

// dX[n,c,h,w] (+)= sum over the taps that reach (h, w) of W[c][kh][kw] * dz[n,c,ho,wo],
// ho = (h + P - kh*D) / S when that divides exactly and lands inside the output.
template <int K>
__global__ __launch_bounds__(kThreads) void dwise_dx(ConvGeom g, const float* __restrict__ wt,
                                                     const float* __restrict__ dz,
                                                     float* __restrict__ dx, int accumulate) {
  const int64_t total = (int64_t)g.N * g.C * g.HW;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * kThreads) {
    const int64_t plane = e / g.HW;   // n * C + c
    const int r = (int)(e - plane * g.HW);
    const int c = (int)(plane % g.C);
    const int h = r / g.W, w = r - h * g.W;
    const float* dzp = dz + plane * g.OHW;
    const float* wp = wt + (int64_t)c * K * K;
    float acc = 0.f;
#pragma unroll
    for (int kh = 0; kh < K; ++kh) {
      const int th = h + g.P - kh * g.D;
      if (th < 0 || th % g.S) continue;
      const int ho = th / g.S;
      if (ho >= g.OH) continue;
#pragma unroll
      for (int kw = 0; kw < K; ++kw) {
        const int tw = w + g.P - kw * g.D;
        if (tw < 0 || tw % g.S) continue;
        const int wo = tw / g.S;
        if (wo >= g.OW) continue;
        acc += wp[kh * K + kw] * dzp[ho * g.OW + wo];
      }
    }
    dx[e] = accumulate ? dx[e] + acc : acc;
  }
}

// ---------------------------------------------------------------------------
// Planes that fit in LDS (an x and a dz plane together at most kDwPlane floats,
// 48 KB): one work-group stages whole planes once with coalesced loads and reads
// every tap from LDS.  The LDS is sized to the planes (dynamic), so small planes
// leave room for several work-groups per CU.
// ---------------------------------------------------------------------------
constexpr int kDwPlane = 12288;

static bool dwise_lds_ok(const ConvGeom& g) { return g.HW + g.OHW <= kDwPlane; }

// dX: work-group = one (image, channel) plane.
template <int K>
__global__ __launch_bounds__(kThreads) void dwise_dx_lds(ConvGeom g, const float* __restrict__ wt,
                                                         const float* __restrict__ dz,
                                                         float* __restrict__ dx, int accumulate) {
  extern __shared__ float zs[];     // the dz plane, OHW floats
  const int64_t plane = blockIdx.x;   // n * C + c
  const int c = (int)(plane % g.C);
  const float* dzp = dz + plane * g.OHW;
  for (int e = threadIdx.x; e < g.OHW; e += kThreads) zs[e] = dzp[e];
  float wk[K * K];
#pragma unroll
  for (int t = 0; t < K * K; ++t) wk[t] = wt[(int64_t)c * K * K + t];
  __syncthreads();
  float* dxp = dx + plane * g.HW;
  if (g.S == 1 && g.W <= kThreads) {
    // every tap lands on an output position: no phase test; each thread keeps one column
    // and walks every R-th row (R = rows per pass), so no index division per element
    const int R = kThreads / g.W, r0 = threadIdx.x / g.W, w = threadIdx.x - r0 * g.W;
    if (r0 >= R) return;
    for (int h = r0; h < g.H; h += R) {
      float acc = 0.f;
#pragma unroll
      for (int kh = 0; kh < K; ++kh) {
        const int ho = h + g.P - kh * g.D;
        if ((unsigned)ho >= (unsigned)g.OH) continue;
#pragma unroll
        for (int kw = 0; kw < K; ++kw) {
          const int wo = w + g.P - kw * g.D;
          if ((unsigned)wo < (unsigned)g.OW) acc += wk[kh * K + kw] * zs[ho * g.OW + wo];
        }
      }
      const int e = h * g.W + w;
      dxp[e] = accumulate ? dxp[e] + acc : acc;
    }
    return;
  }
  if (g.S == 1) {   // every tap lands on an output position: no phase test, no division
    for (int e = threadIdx.x; e < g.HW; e += kThreads) {
      const int h = e / g.W, w = e - h * g.W;
      float acc = 0.f;
#pragma unroll
      for (int kh = 0; kh < K; ++kh) {
        const int ho = h + g.P - kh * g.D;
        if ((unsigned)ho >= (unsigned)g.OH) continue;
#pragma unroll
        for (int kw = 0; kw < K; ++kw) {
          const int wo = w + g.P - kw * g.D;
          if ((unsigned)wo < (unsigned)g.OW) acc += wk[kh * K + kw] * zs[ho * g.OW + wo];
        }
      }
      dxp[e] = accumulate ? dxp[e] + acc : acc;
    }
    return;
  }
  for (int e = threadIdx.x; e < g.HW; e += kThreads) {
    const int h = e / g.W, w = e - h * g.W;
    float acc = 0.f;
#pragma unroll
    for (int kh = 0; kh < K; ++kh) {
      const int th = h + g.P - kh * g.D;
      if (th < 0 || th % g.S) continue;
      const int ho = th / g.S;
      if (ho >= g.OH) continue;
#pragma unroll
      for (int kw = 0; kw < K; ++kw) {
        const int tw = w + g.P - kw * g.D;
        if (tw < 0 || tw % g.S) continue;
        const int wo = tw / g.S;
        if (wo >= g.OW) continue;
        acc += wk[kh * K + kw] * zs[ho * g.OW + wo];
      }
    }
    dxp[e] = accumulate ? dxp[e] + acc : acc;
  }
}

// dW partial sums: work-group (c, segment) walks the images n0 .. n1-1 of its
// segment, staging each image's x and dz planes of channel c in LDS.
template <int K>
__global__ __launch_bounds__(kThreads) void dwise_dw_lds(ConvGeom g, const float* __restrict__ x,
                                                         const float* __restrict__ dz,
                                                         float* __restrict__ part, int nseg,
                                                         int per_seg) {
  extern __shared__ float xz[];     // the x plane (HW floats), then the dz plane
  float* xs = xz;
  float* zs = xz + g.HW;
  const int c = blockIdx.x / nseg, sg = blockIdx.x % nseg;
  const int n0 = sg * per_seg, n1 = min(g.N, n0 + per_seg);
  float acc[K * K];
#pragma unroll
  for (int t = 0; t < K * K; ++t) acc[t] = 0.f;
  for (int n = n0; n < n1; ++n) {
    const float* xp = x + ((int64_t)n * g.C + c) * g.HW;
    const float* dzp = dz + ((int64_t)n * g.C + c) * g.OHW;
    __syncthreads();   // the previous image's reads are done
    for (int e = threadIdx.x; e < g.HW; e += kThreads) xs[e] = xp[e];
    for (int e = threadIdx.x; e < g.OHW; e += kThreads) zs[e] = dzp[e];
    __syncthreads();
    // each thread keeps one output column and walks every R-th output row (R = rows per
    // pass; OW <= 256), else the flat walk with a division per position
    auto one = [&](int ho, int wo) {
      const float d = zs[ho * g.OW + wo];
      const int h0 = ho * g.S - g.P, w0 = wo * g.S - g.P;
#pragma unroll
      for (int kh = 0; kh < K; ++kh) {
        const int h = h0 + kh * g.D;
        const bool hv = (unsigned)h < (unsigned)g.H;
#pragma unroll
        for (int kw = 0; kw < K; ++kw) {
          const int w = w0 + kw * g.D;
          if (hv && (unsigned)w < (unsigned)g.W) acc[kh * K + kw] += d * xs[h * g.W + w];
        }
      }
    };
    if (g.OW <= kThreads) {
      const int R = kThreads / g.OW, r0 = threadIdx.x / g.OW, wo = threadIdx.x - r0 * g.OW;
      if (r0 < R)
        for (int ho = r0; ho < g.OH; ho += R) one(ho, wo);
    } else {
      for (int q = threadIdx.x; q < g.OHW; q += kThreads) {
        const int ho = q / g.OW;
        one(ho, q - ho * g.OW);
      }
    }
  }
  __shared__ float red[4];
#pragma unroll
  for (int t = 0; t < K * K; ++t) {
    const float v = block_sum_256(acc[t], red);
    if (threadIdx.x == 0) part[((int64_t)c * nseg + sg) * (K * K) + t] = v;
  }
}

size_t conv_depthwise_workspace(const ConvGeom& g) {
  const DwiseSeg s = dwise_plan(g);
  return (size_t)g.C * s.nseg * g.K * g.K * sizeof(float);
}

int launch_depthwise_dw(const ConvGeom& g, const float* x, const float* dz, float* dw, float* ws,
                        hipStream_t st) {
  if (dwise_lds_ok(g)) {
    // segments of whole images, no more than the streaming plan's (its workspace)
    const int nseg = std::max(1, std::min(dwise_plan(g).nseg, g.N));
    const int per_seg = (int)ceil_div(g.N, nseg);
    const int nseg2 = (int)ceil_div(g.N, per_seg);
    const unsigned blocks = (unsigned)((int64_t)g.C * nseg2);
    const size_t lds = (size_t)(g.HW + g.OHW) * sizeof(float);
#define CBB_DWL(K_)                                                                          \
  case K_:                                                                                   \
    dwise_dw_lds<K_><<<blocks, kThreads, lds, st>>>(g, x, dz, ws, nseg2, per_seg);           \
    break;
    switch (g.K) {
      CBB_DWL(1) CBB_DWL(2) CBB_DWL(3) CBB_DWL(4) CBB_DWL(5) CBB_DWL(6) CBB_DWL(7)
    }
#undef CBB_DWL
    const int rc = check_launch("dwise_dw_lds", st);
    if (rc) return rc;
    dwise_dw_fold<<<(unsigned)g.C, 64, 0, st>>>(ws, nseg2, g.K * g.K, dw);
    return check_launch("dwise_dw_fold", st);
  }
  const DwiseSeg s = dwise_plan(g);
  const unsigned blocks = (unsigned)((int64_t)g.C * s.nseg);
#define CBB_DWW(K_)                                                                        \
  case K_:                                                                                 \
    dwise_dw_partial<K_><<<blocks, kThreads, 0, st>>>(g, x, dz, ws, s.nseg, s.seglen);     \
    break;
  switch (g.K) {
    CBB_DWW(1) CBB_DWW(2) CBB_DWW(3) CBB_DWW(4) CBB_DWW(5) CBB_DWW(6) CBB_DWW(7)
  }
#undef CBB_DWW
  const int rc = check_launch("dwise_dw_partial", st);
  if (rc) return rc;
  dwise_dw_fold<<<(unsigned)g.C, 64, 0, st>>>(ws, s.nseg, g.K * g.K, dw);
  return check_launch("dwise_dw_fold", st);
}

int launch_depthwise_dx(const ConvGeom& g, const float* wt, const float* dz, float* dx,
                        int accumulate, hipStream_t st) {
  if (dwise_lds_ok(g)) {
    const unsigned blocks = (unsigned)((int64_t)g.N * g.C);
    const size_t lds = (size_t)g.OHW * sizeof(float);
#define CBB_DXL(K_)                                                                          \
  case K_:                                                                                   \
    dwise_dx_lds<K_><<<blocks, kThreads, lds, st>>>(g, wt, dz, dx, accumulate);              \
    break;
    switch (g.K) {
      CBB_DXL(1) CBB_DXL(2) CBB_DXL(3) CBB_DXL(4) CBB_DXL(5) CBB_DXL(6) CBB_DXL(7)
    }
#undef CBB_DXL
    return check_launch("dwise_dx_lds", st);
  }
  const int64_t total = (int64_t)g.N * g.C * g.HW;
  const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(total, kThreads), 16384);
#define CBB_DWX(K_)                                                                   \
  case K_:                                                                            \
    dwise_dx<K_><<<blocks, kThreads, 0, st>>>(g, wt, dz, dx, accumulate);             \
    break;
  switch (g.K) {
    CBB_DWX(1) CBB_DWX(2) CBB_DWX(3) CBB_DWX(4) CBB_DWX(5) CBB_DWX(6) CBB_DWX(7)
  }
#undef CBB_DWX
  return check_launch("dwise_dx", st);
}

}  // namespace cbb
