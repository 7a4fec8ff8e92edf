// layers.hip -- the non-convolution steps of the backward pass: shortcut,
// route, upsample, max-pool, softmax-with-loss and inner product.
//
// "YOLOv3 backpropagation: full-flow source analysis" (suzhouguqin.com):
//   section 5 backward_shortcut_layer (axpy + shortcut_cpu, s1 = 1, s2 = beta),
//   section 6 backward_route_layer (per input, per image axpy of a slice).
// "Caffe source study ch.4 (5): the LeNet backward pass" (csdndocs.com):
//   layer 9 SoftmaxWithLoss (prob - onehot, times loss_weight / count),
//   layer 8 InnerProduct (dW += delta^T X, db += delta^T 1, dX = delta W),
//   layer 5 Pooling MAX (bottom_diff = 0; bottom_diff[mask] += top_diff).
#include "cbb_internal.h"

namespace cbb {

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

static unsigned grid_for(int64_t work) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(ceil_div(work, kThreads), 16384));
}

// --------------------------------------------------------------- shortcut
__global__ __launch_bounds__(kThreads) void shortcut_kernel(int64_t count, float alpha, float beta,
                                                            const float* __restrict__ delta,
                                                            float* __restrict__ d_main,
                                                            float* __restrict__ d_from, int vec) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  int64_t tail = 0;
  if (vec) {
    const int64_t n4 = count >> 2;
    for (int64_t i = i0; i < n4; i += stride) {
      const float4 d = reinterpret_cast<const float4*>(delta)[i];
      float4 m = reinterpret_cast<float4*>(d_main)[i];
      float4 f = reinterpret_cast<float4*>(d_from)[i];
      m.x += alpha * d.x; m.y += alpha * d.y; m.z += alpha * d.z; m.w += alpha * d.w;
      f.x += beta * d.x;  f.y += beta * d.y;  f.z += beta * d.z;  f.w += beta * d.w;
      reinterpret_cast<float4*>(d_main)[i] = m;
      reinterpret_cast<float4*>(d_from)[i] = f;
    }
    tail = 4 * n4;
  }
  for (int64_t i = tail + i0; i < count; i += stride) {
    d_main[i] += alpha * delta[i];
    d_from[i] += beta * delta[i];
  }
}

// Shapes that differ: d_from[b, k, j*sample, i*sample] += beta * delta[b, k, j*stride,
// i*stride] over the smaller shape (one thread per term; the targets are distinct),
// and d_main += alpha * delta over the whole delta.
__global__ __launch_bounds__(kThreads) void shortcut_resize_kernel(
    int batch, int w1, int h1, int c1, int w2, int h2, int c2, int stride, int sample, int minw,
    int minh, int minc, float beta, const float* __restrict__ delta, float* __restrict__ d_from) {
  const int64_t total = (int64_t)batch * minc * minh * minw;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * kThreads) {
    const int i = (int)(e % minw);
    const int64_t r = e / minw;
    const int j = (int)(r % minh);
    const int64_t r2 = r / minh;
    const int k = (int)(r2 % minc), b = (int)(r2 / minc);
    const int64_t out = i * sample + (int64_t)w2 * (j * sample + (int64_t)h2 * (k + (int64_t)c2 * b));
    const int64_t add = i * stride + (int64_t)w1 * (j * stride + (int64_t)h1 * (k + (int64_t)c1 * b));
    d_from[out] += beta * delta[add];
  }
}

__global__ __launch_bounds__(kThreads) void axpy_kernel(int64_t count, float alpha,
                                                        const float* __restrict__ x,
                                                        float* __restrict__ y) {
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < count;
       e += (int64_t)gridDim.x * kThreads)
    y[e] += alpha * x[e];
}

int launch_shortcut_resize(int batch, int w1, int h1, int c1, int w2, int h2, int c2, float alpha,
                           float beta, const float* delta, float* d_main, float* d_from,
                           hipStream_t st) {
  const int stride = std::max(1, w1 / w2), sample = std::max(1, w2 / w1);
  const int minw = std::min(w1, w2), minh = std::min(h1, h2), minc = std::min(c1, c2);
  if (d_main) {
    const int64_t n1 = (int64_t)batch * c1 * h1 * w1;
    axpy_kernel<<<grid_for(n1), kThreads, 0, st>>>(n1, alpha, delta, d_main);
    const int rc = check_launch("axpy_kernel", st);
    if (rc) return rc;
  }
  shortcut_resize_kernel<<<grid_for((int64_t)batch * minc * minh * minw), kThreads, 0, st>>>(
      batch, w1, h1, c1, w2, h2, c2, stride, sample, minw, minh, minc, beta, delta, d_from);
  return check_launch("shortcut_resize_kernel", st);
}

// ------------------------------------------------------------- softmax
// dx[i,c,k] = (dy[i,c,k] - sum_c' dy[i,c',k] y[i,c',k]) * y[i,c,k] (Caffe's
// SoftmaxLayer Backward_cpu).  Contiguous rows (inner = 1): one wave per row,
// the dot summed by a fixed butterfly; otherwise a work-group per 16 positions k
// with the channels split over slices.  Every element's dy is read before any
// thread writes dx (the dot is complete, behind a barrier, before the writes), so
// dx may equal dy.
__global__ __launch_bounds__(kThreads) void softmax_bwd_rows(int outer, int channels,
                                                             const float* __restrict__ y,
                                                             const float* dy, float* dx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= outer) return;
  const float* yr = y + row * channels;
  const float* dr = dy + row * channels;
  float dot = 0.f;
  for (int c = lane; c < channels; c += 64) dot += dr[c] * yr[c];
  dot = wave_sum(dot);
  float* xr = dx + row * channels;
  for (int c = lane; c < channels; c += 64) xr[c] = (dr[c] - dot) * yr[c];
}

// Strided layout (inner > 1): a work-group takes 16 consecutive positions k of one
// outer index and splits the channels over 16 slices (thread = (slice, k)); the
// 16 slice sums of each position are added in slice order through LDS.
constexpr int kSmK = 16, kSmSlices = kThreads / kSmK;
__global__ __launch_bounds__(kThreads) void softmax_bwd_strided(int outer, int channels,
                                                                int64_t inner, int64_t ktiles,
                                                                const float* __restrict__ y,
                                                                const float* dy, float* dx) {
  __shared__ float part[kSmSlices][kSmK];
  const int kl = threadIdx.x % kSmK, sl = threadIdx.x / kSmK;
  const int64_t i = blockIdx.x / ktiles, k = (blockIdx.x % ktiles) * kSmK + kl;
  const bool kv = k < inner;
  const int64_t base = i * channels * inner + k;
  float dot = 0.f;
  if (kv)
    for (int c = sl; c < channels; c += kSmSlices) dot += dy[base + c * inner] * y[base + c * inner];
  part[sl][kl] = dot;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int q = 0; q < kSmSlices; ++q) tot += part[q][kl];
  if (!kv) return;
  for (int c = sl; c < channels; c += kSmSlices) {
    const int64_t e = base + c * inner;
    dx[e] = (dy[e] - tot) * y[e];
  }
}

int launch_softmax_backward(int outer, int channels, int64_t inner, const float* y,
                            const float* dy, float* dx, hipStream_t st) {
  if (inner == 1) {
    softmax_bwd_rows<<<(unsigned)ceil_div(outer, kThreads / 64), kThreads, 0, st>>>(outer, channels,
                                                                                 y, dy, dx);
    return check_launch("softmax_bwd_rows", st);
  }
  const int64_t ktiles = ceil_div(inner, kSmK);
  softmax_bwd_strided<<<(unsigned)(outer * ktiles), kThreads, 0, st>>>(outer, channels, inner,
                                                                       ktiles, y, dy, dx);
  return check_launch("softmax_bwd_strided", st);
}

int launch_shortcut(int64_t count, float alpha, float beta, const float* delta, float* d_main,
                    float* d_from, hipStream_t st) {
  const int vec = aligned16(delta) && aligned16(d_main) && aligned16(d_from);
  shortcut_kernel<<<grid_for(vec ? ceil_div(count, 4) : count), kThreads, 0, st>>>(
      count, alpha, beta, delta, d_main, d_from, vec);
  return check_launch("shortcut_kernel", st);
}

// --------------------------------------------------------------- route
// d_in[t][j*size_t + e] += delta[j*outputs + off_t + e] for every image j and e < size_t:
// one pass over the columns of delta that up to kRouteMax inputs cover (column e of that
// span belongs to the last input whose offset in it is <= e).  vec: every size a multiple
// of 4 (so are the offsets and `outputs`) and the tensors 16-byte aligned; then indices
// count 16-byte units.
constexpr int kRouteMax = 8;
struct RouteArgs {
  int n;
  int64_t size[kRouteMax], off[kRouteMax];
  float* d[kRouteMax];
};
__global__ __launch_bounds__(kThreads) void route_kernel(int batch, int64_t outputs, int64_t span,
                                                         const float* __restrict__ delta,
                                                         RouteArgs a, int vec) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int u = vec ? 4 : 1;
  const int64_t spu = span / u, outu = outputs / u, total = (int64_t)batch * spu;
  for (int64_t i = i0; i < total; i += stride) {
    const int64_t j = i / spu, e = i - j * spu;
    int t = 0;
#pragma unroll
    for (int k = 1; k < kRouteMax; ++k)
      if (k < a.n && a.off[k] / u <= e) t = k;
    const int64_t dst = j * (a.size[t] / u) + e - a.off[t] / u, src = j * outu + e;
    if (vec) {
      const float4 d = reinterpret_cast<const float4*>(delta)[src];
      float4* p = reinterpret_cast<float4*>(a.d[t]) + dst;
      float4 v = *p;
      v.x += d.x; v.y += d.y; v.z += d.z; v.w += d.w;
      *p = v;
    } else {
      a.d[t][dst] += delta[src];
    }
  }
}

int launch_route(int batch, int n_in, const int64_t* sizes, const float* delta,
                 float* const* d_in, hipStream_t st) {
  // n_in <= kRouteMax (checked by the API): one launch over the whole route delta
  RouteArgs a{};
  a.n = n_in;
  int64_t outputs = 0;
  bool vec = aligned16(delta);
  for (int k = 0; k < n_in; ++k) {
    a.size[k] = sizes[k];
    a.off[k] = outputs;
    a.d[k] = d_in[k];
    vec = vec && sizes[k] % 4 == 0 && aligned16(d_in[k]);
    outputs += sizes[k];
  }
  const int64_t work = (int64_t)batch * (vec ? outputs / 4 : outputs);
  route_kernel<<<grid_for(work), kThreads, 0, st>>>(batch, outputs, outputs, delta, a,
                                                    vec ? 1 : 0);
  return check_launch("route_kernel", st);
}

// --------------------------------------------------------------- upsample
// dx[p, r, q] += sum_{a,b < scale} delta[p, r*scale + a, q*scale + b]; one thread per small pixel.
__global__ __launch_bounds__(kThreads) void upsample_bwd_kernel(int64_t planes, int h, int w,
                                                                int scale,
                                                                const float* __restrict__ delta,
                                                                float* __restrict__ dx) {
  const int64_t total = planes * h * w;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int W = w * scale;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += stride) {
    const int64_t pl = i / ((int64_t)h * w);
    const int rq = (int)(i - pl * h * w);
    const int r = rq / w, q = rq - r * w;
    const float* src = delta + (pl * h * scale + (int64_t)r * scale) * W + (int64_t)q * scale;
    float acc = 0.f;
    for (int a = 0; a < scale; ++a)
      for (int b = 0; b < scale; ++b) acc += src[(int64_t)a * W + b];
    dx[i] += acc;
  }
}

int launch_upsample(int n, int c, int h, int w, int scale, const float* delta, float* dx,
                    hipStream_t st) {
  const int64_t planes = (int64_t)n * c;
  upsample_bwd_kernel<<<grid_for(planes * h * w), kThreads, 0, st>>>(planes, h, w, scale, delta,
                                                                     dx);
  return check_launch("upsample_bwd_kernel", st);
}

// --------------------------------------------------------------- max pool
// Gather form: every bottom pixel sums, in (ph, pw) order, the deltas of the
// windows that contain it and whose mask names it.  Writes every dx element
// once (no separate clearing pass, no atomics).
__global__ __launch_bounds__(kThreads) void maxpool_bwd_kernel(int64_t planes, int ih, int iw,
                                                               int oh, int ow, int k, int s,
                                                               const int* __restrict__ idx,
                                                               const float* __restrict__ delta,
                                                               float* __restrict__ dx) {
  const int64_t total = planes * ih * iw;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += stride) {
    const int64_t pl = i / ((int64_t)ih * iw);
    const int pix = (int)(i - pl * ih * iw);
    const int h = pix / iw, w = pix - h * iw;
    // windows ph with ph*s <= h <= ph*s + k - 1
    const int ph0 = h >= k ? (h - k) / s + 1 : 0, ph1 = min(h / s, oh - 1);
    const int pw0 = w >= k ? (w - k) / s + 1 : 0, pw1 = min(w / s, ow - 1);
    const int64_t base = pl * oh * ow;
    float acc = 0.f;
    for (int ph = ph0; ph <= ph1; ++ph)
      for (int pw = pw0; pw <= pw1; ++pw) {
        const int64_t o = base + (int64_t)ph * ow + pw;
        if (idx[o] == pix) acc += delta[o];
      }
    dx[i] = acc;
  }
}

int launch_maxpool(int n, int c, int ih, int iw, int k, int s, const int32_t* idx,
                   const float* delta, float* dx, hipStream_t st) {
  const int oh = (ih - k) / s + 1, ow = (iw - k) / s + 1;
  const int64_t planes = (int64_t)n * c;
  maxpool_bwd_kernel<<<grid_for(planes * ih * iw), kThreads, 0, st>>>(planes, ih, iw, oh, ow, k,
                                                                      s, idx, delta, dx);
  return check_launch("maxpool_bwd_kernel", st);
}

// --------------------------------------------------------------- softmax loss
__global__ __launch_bounds__(kThreads) void softmax_loss_bwd_kernel(
    int batch, int classes, const float* __restrict__ prob, const int32_t* __restrict__ labels,
    float scale, float* __restrict__ dlogits, int32_t* __restrict__ bad,
    int32_t* __restrict__ dev_err) {
  const int64_t total = (int64_t)batch * classes;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += stride) {
    const int b = (int)(i / classes), j = (int)(i - (int64_t)b * classes);
    const int lab = labels[b];
    const bool valid = lab >= 0 && lab < classes;
    float p = prob[i];
    if (valid && j == lab) p -= 1.f;
    dlogits[i] = p * scale;
    if (!valid && j == 0) {
      if (bad) atomicAdd(bad, 1);
      atomicOr(dev_err, CBB_DEVERR_LABEL);
    }
  }
}

int launch_softmax_loss(int batch, int classes, const float* prob, const int32_t* labels,
                        float loss_weight, float* dlogits, int32_t* bad, hipStream_t st) {
  int32_t* dev_err = device_error_word();
  if (!dev_err) return CBB_EHIP;
  softmax_loss_bwd_kernel<<<grid_for((int64_t)batch * classes), kThreads, 0, st>>>(
      batch, classes, prob, labels, loss_weight / (float)batch, dlogits, bad, dev_err);
  return check_launch("softmax_loss_bwd_kernel", st);
}

// --------------------------------------------------------------- inner product
// C[m][n] (+)= sum_k A(m,k) B(k,n), A(m,k) = A[m*sam + k*sak], B(k,n) = B[k*sbk + n*sbn],
// C[m*ldc + n].  64x64 tiles on the 32x32x2 fp32 matrix cores, K in steps of 32.
// Batched over grid y: problem b reads B + b*sbb and writes C + b*scb (A shared);
// GemmArgs is declared in cbb_internal.h.

// TS = TileShape<2, 2, 1> (64x64 tiles), or TileShape<1, 1, 4> (32x32 tiles,
// the four waves splitting each K tile) for small outputs with a long K.
template <class TS>
__global__ __launch_bounds__(kThreads) void strided_gemm_kernel(GemmArgs a, int tiles_n) {
  __shared__ float lds[TS::LDS_FLOATS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % TS::WM, wn = (wave / TS::WM) % TS::WN, wk = wave / (TS::WM * TS::WN);
  const int m0 = (blockIdx.x / tiles_n) * TS::BM, n0 = (blockIdx.x % tiles_n) * TS::BN;
  a.B += blockIdx.y * a.sbb;
  a.C += blockIdx.y * a.scb;
  // Register-prefetched K tiles (two ahead, see gemm_mainloop); out-of-range
  // elements read a clamped address and are zeroed at the LDS store, so the
  // loads stay in flight during the matrix-core work.
  float ra[TS::A_PER_T], rb[TS::B_PER_T];
  uint32_t am = 0, bm = 0;
  auto load = [&](int64_t k0) {
    am = 0;
    bm = 0;
#pragma unroll
    for (int r = 0; r < TS::A_PER_T; ++r) {
      const int e = tid + kThreads * r;
      const int k = e % TS::BK, m = e / TS::BK;
      const int gm = m0 + m, gk = (int)k0 + k;
      const bool ok = gm < a.M && gk < a.K;
      ra[r] = a.A[ok ? (int64_t)gm * a.sam + (int64_t)gk * a.sak : 0];
      am |= (uint32_t)ok << r;
    }
#pragma unroll
    for (int r = 0; r < TS::B_PER_T; ++r) {
      const int e = tid + kThreads * r;
      const int n = e % TS::BN, k = e / TS::BN;
      const int gn = n0 + n, gk = (int)k0 + k;
      const bool ok = gn < a.N && gk < a.K;
      rb[r] = a.B[ok ? (int64_t)gk * a.sbk + (int64_t)gn * a.sbn : 0];
      bm |= (uint32_t)ok << r;
    }
  };
  auto store = [&](float* buf) {
    float* As = buf;
    float* Bs = buf + TS::BK * TS::LDA;
#pragma unroll
    for (int r = 0; r < TS::A_PER_T; ++r) {
      const int e = tid + kThreads * r;
      As[(e % TS::BK) * TS::LDA + e / TS::BK] = ((am >> r) & 1u) ? ra[r] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < TS::B_PER_T; ++r) {
      const int e = tid + kThreads * r;
      Bs[(e / TS::BN) * TS::LDB + e % TS::BN] = ((bm >> r) & 1u) ? rb[r] : 0.f;
    }
  };
  Acc<TS> acc;
  acc.zero();
  gemm_mainloop<TS>(lds, 0, a.K, load, store, acc, wm, wn, wk, lane);
  reduce_wk<TS>(acc, lds, wm, wn, wk, lane);
  if (wk != 0) return;
#pragma unroll
  for (int i = 0; i < TS::RM; ++i)
#pragma unroll
    for (int j = 0; j < TS::RN; ++j) {
      const int n = n0 + acc_n0<TS>(wn, j) + acc_col(lane);
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + acc_m0<TS>(wm, i) + acc_row(r, lane);
        if (m < a.M) {
          float* c = a.C + (int64_t)m * a.ldc + n;
          *c = a.accumulate ? *c + acc.v[i][j][r] : acc.v[i][j][r];
        }
      }
    }
}

int launch_gemm(const GemmArgs& a, hipStream_t st, int batch) {
  const int64_t tiles64 = ceil_div(a.M, 64) * ceil_div(a.N, 64) * batch;
  if (tiles64 < 64 && a.K >= 256) {
    // few 64x64 tiles over a long K: 32x32 tiles, K split over the four waves
    using TS = TileShape<1, 1, 4>;
    const int tiles_n = (int)ceil_div(a.N, 32);
    const int tiles = (int)ceil_div(a.M, 32) * tiles_n;
    strided_gemm_kernel<TS><<<dim3(tiles, batch), kThreads, 0, st>>>(a, tiles_n);
  } else {
    using TS = TileShape<2, 2, 1>;
    const int tiles_n = (int)ceil_div(a.N, 64);
    const int tiles = (int)ceil_div(a.M, 64) * tiles_n;
    strided_gemm_kernel<TS><<<dim3(tiles, batch), kThreads, 0, st>>>(a, tiles_n);
  }
  return check_launch("strided_gemm_kernel", st);
}

// db[o] += sum over the batch of delta[b][o], batch rows in order.
__global__ __launch_bounds__(kThreads) void fc_bias_kernel(int batch, int out,
                                                           const float* __restrict__ delta,
                                                           float* __restrict__ db) {
  const int o = blockIdx.x * kThreads + threadIdx.x;
  if (o >= out) return;
  // batch rows in order, 16 loads in flight before each group's adds
  float s = 0.f;
  for (int b0 = 0; b0 < batch; b0 += 16) {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = delta[(int64_t)min(b0 + k, batch - 1) * out + o];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (b0 + k < batch) s += v[k];
  }
  db[o] += s;
}

int launch_fc(int batch, int in_dim, int out_dim, const float* x, const float* w,
              const float* delta, float* dw, float* db, float* dx, int dx_accumulate,
              hipStream_t st) {
  // dW (out x in) += delta^T (out x batch) . X (batch x in)
  GemmArgs gw{out_dim, in_dim, batch, delta, 1, out_dim, x, in_dim, 1, dw, in_dim, 1};
  int rc = launch_gemm(gw, st);
  if (rc) return rc;
  if (db) {
    fc_bias_kernel<<<(unsigned)ceil_div(out_dim, kThreads), kThreads, 0, st>>>(batch, out_dim,
                                                                               delta, db);
    rc = check_launch("fc_bias_kernel", st);
    if (rc) return rc;
  }
  if (dx) {
    // dX (batch x in) (+)= delta (batch x out) . W (out x in)
    GemmArgs gx{batch, in_dim, out_dim, delta, out_dim, 1, w, in_dim, 1, dx, in_dim,
                dx_accumulate};
    rc = launch_gemm(gx, st);
  }
  return rc;
}

}  // namespace cbb

namespace cbb {

// --------------------------------------------------------------- parameter update
// Gradient descent after the backward pass, once per full batch (the pages' update
// step; see cbb_sgd_update): u = dw + decay*batch*w; w -= lr/batch * u;
// dw = momentum * u.  One read and one write of w and dw per element, 16-byte
// accesses, the ragged tail element by element.
__global__ __launch_bounds__(kThreads) void sgd_update_kernel(int64_t n, int vec, float kdecay,
                                                              float step, float momentum,
                                                              float* __restrict__ w,
                                                              float* __restrict__ dw) {
  const int64_t n4 = vec ? n >> 2 : 0;   // 16-byte accesses need 16-byte aligned w and dw
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    float4 a = reinterpret_cast<float4*>(w)[i];
    float4 g = reinterpret_cast<float4*>(dw)[i];
    g.x += kdecay * a.x;
    g.y += kdecay * a.y;
    g.z += kdecay * a.z;
    g.w += kdecay * a.w;
    a.x -= step * g.x;
    a.y -= step * g.y;
    a.z -= step * g.z;
    a.w -= step * g.w;
    reinterpret_cast<float4*>(w)[i] = a;
    reinterpret_cast<float4*>(dw)[i] = make_float4(momentum * g.x, momentum * g.y,
                                                   momentum * g.z, momentum * g.w);
  }
  for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    const float u = dw[i] + kdecay * w[i];
    w[i] -= step * u;
    dw[i] = momentum * u;
  }
}

int launch_sgd_update(int64_t n, int batch, float lr, float momentum, float decay, float* w,
                      float* dw, hipStream_t st) {
  const int vec = ((uintptr_t)w % 16 == 0) && ((uintptr_t)dw % 16 == 0);
  const int64_t items = vec ? std::max<int64_t>(n >> 2, 1) : n;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(ceil_div(items, kThreads), 8192));
  sgd_update_kernel<<<(unsigned)blocks, kThreads, 0, st>>>(n, vec, decay * (float)batch,
                                                            lr / (float)batch, momentum, w, dw);
  return check_launch("sgd_update_kernel", st);
}

}  // namespace cbb
