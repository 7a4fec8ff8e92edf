// conv.hip -- weight and input gradients of a convolution as implicit GEMMs on
// the gfx950 fp32 matrix cores, with the im2col / col2im index maps applied
// while staging tiles into LDS (no column buffer is ever written).
//
// Pages: "YOLOv3 backpropagation: full-flow source analysis" (suzhouguqin.com),
// section 3.1 (backward_convolutional_layer: dW = delta x im2col(x)^T with
// beta = 1, dX = col2im(W^T x delta)) and section 3.2 (im2col_cpu/col2im_cpu
// index map, output size (size + 2 pad - k)/stride + 1).
#include "cbb_internal.h"

namespace cbb {

// ---------------------------------------------------------------------------
// Weight gradient.  dW[o][j] = sum_q A[o][q] * B[q][j] with
//   q = (n, ho, wo),  A[o][q] = dz[n][o][ho][wo],
//   j = (i, kh, kw),  B[q][j] = x[n][i][ho*s+kh-p][wo*s+kw-p]  (0 off the image).
// Grid: x = output tiles, y = slices of q (split-K).  With one slice the tile
// is added into dw directly; otherwise each slice writes its partial tile to
// `out` = workspace[slice][o][j] and dw_splitk_reduce adds them up in order.
// ---------------------------------------------------------------------------
template <class TS>
__global__ __launch_bounds__(kThreads) void conv_dw_kernel(ConvGeom g, const float* __restrict__ x,
                                                           const float* __restrict__ dz,
                                                           float* __restrict__ out,
                                                           int64_t k_chunk, int tiles_n,
                                                           int direct) {
  __shared__ float lds[TS::LDS_FLOATS];
  float* As = lds;
  float* Bs = lds + TS::BK * TS::LDA;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % TS::WM, wn = (wave / TS::WM) % TS::WN, wk = wave / (TS::WM * TS::WN);
  const int m0 = (blockIdx.x / tiles_n) * TS::BM, n0 = (blockIdx.x % tiles_n) * TS::BN;
  const int64_t kbeg = (int64_t)blockIdx.y * k_chunk;
  const int64_t kend = min(g.Q, kbeg + k_chunk);

  constexpr int RSTEP = kThreads / TS::BK;
  const int qi = tid % TS::BK;    // K row (q) this thread stages
  const int rbase = tid / TS::BK; // first M / N index it stages, then +RSTEP

  // Fixed B columns of this thread: tap offsets inside an image.
  int boff[TS::B_PER_T], bkh[TS::B_PER_T], bkw[TS::B_PER_T];
#pragma unroll
  for (int r = 0; r < TS::B_PER_T; ++r) {
    const int j = n0 + rbase + RSTEP * r;
    const int kk = g.K * g.K;
    const int i = j / kk, rem = j - i * kk;
    const int kh = rem / g.K, kw = rem - kh * g.K;
    if (j < g.J) {
      boff[r] = i * g.HW + kh * g.W + kw;
      bkh[r] = kh;
      bkw[r] = kw;
    } else {  // column beyond J: force the bounds test to fail
      boff[r] = 0;
      bkh[r] = -(1 << 28);
      bkw[r] = 0;
    }
  }

  float ra[TS::A_PER_T], rb[TS::B_PER_T];
  auto load = [&](int64_t k0) {
    const int64_t q = k0 + qi;
    const bool qv = q < kend;
    int b = 0, rem = 0, hb = 0, wb = 0;
    if (qv) {
      b = (int)(q / g.OHW);
      rem = (int)(q - (int64_t)b * g.OHW);
      const int ho = rem / g.OW, wo = rem - ho * g.OW;
      hb = ho * g.S - g.P;
      wb = wo * g.S - g.P;
    }
    const float* db = dz + ((int64_t)b * g.OC) * g.OHW + rem;
#pragma unroll
    for (int r = 0; r < TS::A_PER_T; ++r) {
      const int o = m0 + rbase + RSTEP * r;
      ra[r] = (qv && o < g.OC) ? db[(int64_t)o * g.OHW] : 0.f;
    }
    // x index of (n, i, hb + kh, wb + kw) = image base + boff + hb*W + wb
    const float* xb = x + (int64_t)b * g.C * g.HW;
    const int pbase = hb * g.W + wb;
#pragma unroll
    for (int r = 0; r < TS::B_PER_T; ++r) {
      const int h = hb + bkh[r], w = wb + bkw[r];
      const bool ok = qv && (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
      rb[r] = ok ? xb[boff[r] + pbase] : 0.f;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int r = 0; r < TS::A_PER_T; ++r) As[qi * TS::LDA + rbase + RSTEP * r] = ra[r];
#pragma unroll
    for (int r = 0; r < TS::B_PER_T; ++r) Bs[qi * TS::LDB + rbase + RSTEP * r] = rb[r];
  };

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  if (kbeg < kend) load(kbeg);
  for (int64_t k0 = kbeg; k0 < kend; k0 += TS::BK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + TS::BK < kend) load(k0 + TS::BK);
    mfma_tile<TS>(As, Bs, acc, wm, wn, wk, lane);
  }
  reduce_wk<TS>(acc, lds, wm, wn, wk, lane);
  if (wk == 0) {
    const int j = n0 + wn * 32 + acc_col(lane);
    float* dst = direct ? out : out + (int64_t)blockIdx.y * g.OC * g.J;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int o = m0 + wm * 32 + acc_row(r, lane);
      if (o < g.OC && j < g.J) {
        const int64_t e = (int64_t)o * g.J + j;
        if (direct)
          dst[e] += acc[r];
        else
          dst[e] = acc[r];
      }
    }
  }
}

// dw[e] += sum over slices s (in order) of part[s][e].
__global__ __launch_bounds__(kThreads) void dw_splitk_reduce(float* __restrict__ dw,
                                                             const float* __restrict__ part,
                                                             int splits, int64_t mn) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e >= mn) return;
  float s = 0.f;
  for (int sp = 0; sp < splits; ++sp) s += part[(int64_t)sp * mn + e];
  dw[e] += s;
}

// ---------------------------------------------------------------------------
// Input gradient, gather form of col2im(W^T x delta).  For stride s the input
// pixels split into s*s phases (h mod s, w mod s); inside a phase every pixel
// receives the same set of taps kh = rh + s*th (rh = (ph + p) mod s), and the
// output row it reads is ho = (h + p - kh)/s = hh + bh - th with h = ph + s*hh,
// bh = (ph + p - rh)/s.  Each phase is a dense GEMM
//   dx[i][pix] = sum_kk A[i][kk] * B[kk][pix],   kk = t*OC + o (tap-major),
//   A[i][kk] = W[o][i][kh][kw],  B[kk][pix] = dz[n][o][ho][wo] (0 off the map),
// so no matrix-core work is spent on the stride's empty taps.
// Grid: x = pixel tiles, y = channel tiles, z = phase.
// ---------------------------------------------------------------------------
template <class TS>
__global__ __launch_bounds__(kThreads) void conv_dx_kernel(ConvGeom g, const float* __restrict__ wt,
                                                           const float* __restrict__ dz,
                                                           float* __restrict__ dx,
                                                           int accumulate) {
  static_assert(kThreads % TS::BN == 0 && kThreads % TS::BK == 0, "thread/tile mapping");
  __shared__ float lds[TS::LDS_FLOATS];
  float* As = lds;
  float* Bs = lds + TS::BK * TS::LDA;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % TS::WM, wn = (wave / TS::WM) % TS::WN, wk = wave / (TS::WM * TS::WN);

  const int S = g.S;
  const int ph = blockIdx.z / S, pw = blockIdx.z % S;
  const int HH = (g.H - ph + S - 1) / S, WW = (g.W - pw + S - 1) / S;
  const int npix = g.N * HH * WW;
  const int n0 = blockIdx.x * TS::BN;
  if (n0 >= npix) return;  // this phase has fewer pixels than the grid covers
  const int m0 = blockIdx.y * TS::BM;
  const int rh = (ph + g.P) % S, rw = (pw + g.P) % S;
  const int nkh = rh < g.K ? (g.K - rh + S - 1) / S : 0;
  const int nkw = rw < g.K ? (g.K - rw + S - 1) / S : 0;
  const int bh = (ph + g.P - rh) / S, bw = (pw + g.P - rw) / S;
  const int ntap = nkh * nkw;
  const int KT = g.OC * ntap;

  // B: this thread stages pixel column pcol for K rows krow0 + KSTEP*r.
  constexpr int KSTEP = kThreads / TS::BN;
  const int pcol = tid % TS::BN, krow0 = tid / TS::BN;
  const int pix = n0 + pcol;
  const bool pv = pix < npix;
  int pb = 0, phh = 0, pww = 0;
  if (pv) {
    pb = pix / (HH * WW);
    const int r = pix - pb * HH * WW;
    phh = r / WW;
    pww = r - phh * WW;
  }
  const float* dzb = dz + (int64_t)pb * g.OC * g.OHW;
  const int hob = phh + bh, wob = pww + bw;

  // A: this thread stages K column acol for channel rows m0 + irow0 + ISTEP*r.
  constexpr int ISTEP = kThreads / TS::BK;
  const int acol = tid % TS::BK, irow0 = tid / TS::BK;

  float ra[TS::A_PER_T], rb[TS::B_PER_T];
  auto load = [&](int k0) {
    {  // A = weights
      const int kk = k0 + acol;
      const int t = kk / g.OC, o = kk - t * g.OC;
      const int th = nkw ? t / nkw : 0, tw = t - th * nkw;
      const int kh = rh + S * th, kw = rw + S * tw;
      const bool kv = kk < KT;
      const float* wp = wt + ((int64_t)o * g.C * g.K + kh) * g.K + kw;
#pragma unroll
      for (int r = 0; r < TS::A_PER_T; ++r) {
        const int i = m0 + irow0 + ISTEP * r;
        ra[r] = (kv && i < g.C) ? wp[(int64_t)i * g.K * g.K] : 0.f;
      }
    }
    {  // B = deltas
      int kk = k0 + krow0;
      int t = kk / g.OC, o = kk - t * g.OC;
#pragma unroll
      for (int r = 0; r < TS::B_PER_T; ++r) {
        const int th = nkw ? t / nkw : 0, tw = t - th * nkw;
        const int ho = hob - th, wo = wob - tw;
        const bool ok = pv && (k0 + krow0 + KSTEP * r) < KT && (unsigned)ho < (unsigned)g.OH &&
                        (unsigned)wo < (unsigned)g.OW;
        rb[r] = ok ? dzb[(int64_t)o * g.OHW + ho * g.OW + wo] : 0.f;
        o += KSTEP;
        while (o >= g.OC) {
          o -= g.OC;
          ++t;
        }
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int r = 0; r < TS::A_PER_T; ++r) As[acol * TS::LDA + irow0 + ISTEP * r] = ra[r];
#pragma unroll
    for (int r = 0; r < TS::B_PER_T; ++r) Bs[(krow0 + KSTEP * r) * TS::LDB + pcol] = rb[r];
  };

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  if (KT > 0) load(0);
  for (int k0 = 0; k0 < KT; k0 += TS::BK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + TS::BK < KT) load(k0 + TS::BK);
    mfma_tile<TS>(As, Bs, acc, wm, wn, wk, lane);
  }
  reduce_wk<TS>(acc, lds, wm, wn, wk, lane);
  if (wk == 0) {
    const int p = n0 + wn * 32 + acc_col(lane);
    if (p < npix) {
      const int b = p / (HH * WW);
      const int r2 = p - b * HH * WW;
      const int hh = r2 / WW, ww = r2 - hh * WW;
      const int h = ph + S * hh, w = pw + S * ww;
      float* dst = dx + ((int64_t)b * g.C) * g.HW + h * g.W + w;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = m0 + wm * 32 + acc_row(r, lane);
        if (i < g.C) {
          float* d = dst + (int64_t)i * g.HW;
          *d = accumulate ? *d + acc[r] : acc[r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
ConvGeom make_geom(const cbb_conv_desc& d) {
  ConvGeom g;
  g.N = d.batch;
  g.C = d.in_c;
  g.H = d.in_h;
  g.W = d.in_w;
  g.OC = d.out_c;
  g.K = d.ksize;
  g.S = d.stride;
  g.P = d.pad;
  g.OH = (d.in_h + 2 * d.pad - d.ksize) / d.stride + 1;
  g.OW = (d.in_w + 2 * d.pad - d.ksize) / d.stride + 1;
  g.HW = g.H * g.W;
  g.OHW = g.OH * g.OW;
  g.J = g.C * g.K * g.K;
  g.Q = (int64_t)g.N * g.OHW;
  return g;
}

enum DwShape { DW_64x64 = 0, DW_32x32 = 1, DW_32x64 = 2, DW_64x32 = 3 };

struct DwPlan {
  int shape, bm, bn, bk, tiles_m, tiles_n, splits;
  int64_t k_chunk;
};

static DwPlan plan_dw(const ConvGeom& g) {
  static const int cand[4][3] = {{64, 64, 32}, {32, 32, 128}, {32, 64, 64}, {64, 32, 64}};
  DwPlan best{};
  double best_cost = 1e300;
  for (int s = 0; s < 4; ++s) {
    const int bm = cand[s][0], bn = cand[s][1];
    const double tm = (double)ceil_div(g.OC, bm), tn = (double)ceil_div(g.J, bn);
    // padded matrix-core work, lightly favouring larger tiles (less re-staging)
    const double cost = tm * bm * tn * bn * (1.0 + 0.15 * (64.0 * 64.0) / (bm * bn));
    if (cost < best_cost) {
      best_cost = cost;
      best.shape = s;
      best.bm = bm;
      best.bn = bn;
      best.bk = cand[s][2];
    }
  }
  best.tiles_m = (int)ceil_div(g.OC, best.bm);
  best.tiles_n = (int)ceil_div(g.J, best.bn);
  const int64_t tiles = (int64_t)best.tiles_m * best.tiles_n;
  const int64_t ktiles = ceil_div(g.Q, best.bk);
  int64_t splits = ceil_div(1024, tiles);                  // aim at ~4 work-groups per CU
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, ktiles / 4));  // >= 4 K tiles each
  splits = std::max<int64_t>(1, std::min<int64_t>(splits, 4096));
  int64_t chunk = ceil_div(ktiles, splits) * best.bk;
  best.splits = (int)ceil_div(g.Q, chunk);
  best.k_chunk = chunk;
  return best;
}

size_t conv_dw_workspace(const ConvGeom& g) {
  const DwPlan p = plan_dw(g);
  return p.splits > 1 ? (size_t)p.splits * g.OC * g.J * sizeof(float) : 0;
}

int launch_conv_dw(const ConvGeom& g, const float* x, const float* dz, float* dw, float* ws,
                   hipStream_t st) {
  const DwPlan p = plan_dw(g);
  const int direct = p.splits == 1;
  float* out = direct ? dw : ws;
  dim3 grid(p.tiles_m * p.tiles_n, p.splits);
  switch (p.shape) {
    case DW_64x64:
      conv_dw_kernel<TileShape<2, 2, 1>><<<grid, kThreads, 0, st>>>(g, x, dz, out, p.k_chunk,
                                                                     p.tiles_n, direct);
      break;
    case DW_32x32:
      conv_dw_kernel<TileShape<1, 1, 4>><<<grid, kThreads, 0, st>>>(g, x, dz, out, p.k_chunk,
                                                                     p.tiles_n, direct);
      break;
    case DW_32x64:
      conv_dw_kernel<TileShape<1, 2, 2>><<<grid, kThreads, 0, st>>>(g, x, dz, out, p.k_chunk,
                                                                     p.tiles_n, direct);
      break;
    default:
      conv_dw_kernel<TileShape<2, 1, 2>><<<grid, kThreads, 0, st>>>(g, x, dz, out, p.k_chunk,
                                                                     p.tiles_n, direct);
      break;
  }
  int rc = check_launch("conv_dw_kernel");
  if (rc != CBB_OK || direct) return rc;
  const int64_t mn = (int64_t)g.OC * g.J;
  dw_splitk_reduce<<<(unsigned)ceil_div(mn, kThreads), kThreads, 0, st>>>(dw, ws, p.splits, mn);
  return check_launch("dw_splitk_reduce");
}

int launch_conv_dx(const ConvGeom& g, const float* wt, const float* dz, float* dx, int accumulate,
                   hipStream_t st) {
  const int S = g.S;
  const int maxpix = g.N * ((g.H + S - 1) / S) * ((g.W + S - 1) / S);
  if (g.C <= 32) {
    using TS = TileShape<1, 4, 1>;  // 32 channels x 128 pixels
    dim3 grid((unsigned)ceil_div(maxpix, TS::BN), (unsigned)ceil_div(g.C, TS::BM), S * S);
    conv_dx_kernel<TS><<<grid, kThreads, 0, st>>>(g, wt, dz, dx, accumulate);
  } else {
    using TS = TileShape<2, 2, 1>;  // 64 channels x 64 pixels
    dim3 grid((unsigned)ceil_div(maxpix, TS::BN), (unsigned)ceil_div(g.C, TS::BM), S * S);
    conv_dx_kernel<TS><<<grid, kThreads, 0, st>>>(g, wt, dz, dx, accumulate);
  }
  return check_launch("conv_dx_kernel");
}

}  // namespace cbb
