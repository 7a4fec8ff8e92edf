// conv_fwd.hip -- forward convolution as an implicit GEMM on the gfx950 fp32
// matrix cores, the first half of the conv block's forward (the saved tensors the
// backward reads come from it).
//
// Pages: "YOLOv3 backpropagation: full-flow source analysis" (suzhouguqin.com),
// sections 3.1-3.2: per image, im2col(x) then gemm(W, col) -- here one launch over
// the whole batch with the im2col index map applied while staging (no column
// buffer):
//   z[n][o][q] = sum_j W[o][j] * B[j][q],   j = (i, kh, kw),  q = (ho, wo),
//   B[j][q] = x[n][i][ho*S + kh*D - P][wo*S + kw*D - P]   (0 off the image).
// Groups: the group index is blockIdx.y (group g owns output channels g*OC/G..,
// input channels g*C/G.. and weight block g); ConvGeom holds the group's channel
// counts and the whole tensors' image strides.
#include "cbb_internal.h"

namespace cbb {

// k / d for k < 2^32 / d with one multiply-high: m = ceil(2^32 / d), exact in that
// range (the error of the rounded-up reciprocal stays below 1/d).
struct FastDiv {
  uint32_t m, d;
};
static FastDiv make_fastdiv(uint32_t d) {
  return FastDiv{d == 1 ? 0u : (uint32_t)(((uint64_t)1 << 32) / d + (((uint64_t)1 << 32) % d != 0)), d};
}
__device__ __forceinline__ uint32_t fdiv(uint32_t k, FastDiv f) {
  return f.d == 1 ? k : __umulhi(k, f.m);
}

template <class TS>
__global__ __launch_bounds__(kThreads) void conv_fwd_kernel(ConvGeom g, const float* __restrict__ x,
                                                            const float* __restrict__ wt,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ z, int tiles_m,
                                                            FastDiv div_kk, FastDiv div_k) {
  static_assert(kThreads % TS::BN == 0 && kThreads % TS::BK == 0, "thread/tile mapping");
  // group blockIdx.y (g holds the group's channel counts)
  x += blockIdx.y * g.gx;
  wt += blockIdx.y * g.gw;
  z += blockIdx.y * g.gz;
  if (bias) bias += blockIdx.y * (int64_t)g.OC;
  __shared__ float lds[TS::LDS_FLOATS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % TS::WM, wn = (wave / TS::WM) % TS::WN, wk = wave / (TS::WM * TS::WN);
  // the output-channel tiles of one pixel tile (the same x gathers) run together
  const int m0 = (int)(blockIdx.x % (unsigned)tiles_m) * TS::BM;
  const int64_t n0 = (int64_t)(blockIdx.x / (unsigned)tiles_m) * TS::BN;
  const int KK = g.K * g.K;

  // B: this thread stages pixel column pcol for K rows krow0 + KSTEP*r
  constexpr int KSTEP = kThreads / TS::BN;
  const int pcol = tid % TS::BN, krow0 = tid / TS::BN;
  const int64_t q = n0 + pcol;
  const bool qv = q < g.Q;
  int hb = 0, wb = 0;
  const float* xb = x;
  if (qv) {
    const int b = (int)(q / g.OHW), r = (int)(q - (int64_t)b * g.OHW);
    const int ho = r / g.OW, wo = r - ho * g.OW;
    hb = ho * g.S - g.P;
    wb = wo * g.S - g.P;
    xb = x + (int64_t)b * g.xs;
  }
  // A: this thread stages K column acol for output-channel rows irow0 + ISTEP*r
  constexpr int ISTEP = kThreads / TS::BK;
  const int acol = tid % TS::BK, irow0 = tid / TS::BK;

  // Loads go to registers as they are (out-of-range elements from a clamped valid
  // address); the zero padding is applied at the LDS store, so the loads stay in
  // flight during the matrix-core work.
  static_assert(TS::A_PER_T <= 32 && TS::B_PER_T <= 32, "one mask bit per staged element");
  float ra[TS::A_PER_T], rb[TS::B_PER_T];
  uint32_t am = 0, bm = 0;
  auto load = [&](int64_t k0l) {
    const int k0 = (int)k0l;
    {  // A = weights W[o][j]
      const int j = k0 + acol;
      const bool jv = j < g.J;
      am = 0;
#pragma unroll
      for (int r = 0; r < TS::A_PER_T; ++r) {
        const int o = m0 + irow0 + ISTEP * r;
        const bool ok = jv && o < g.OC;
        ra[r] = wt[ok ? (int64_t)o * g.J + j : 0];
        am |= (uint32_t)ok << r;
      }
    }
    bm = 0;
#pragma unroll
    for (int r = 0; r < TS::B_PER_T; ++r) {  // B = im2col(x)
      const int j = k0 + krow0 + KSTEP * r;
      const int i = (int)fdiv((uint32_t)j, div_kk);
      const int rem = j - i * KK;
      const int kh = (int)fdiv((uint32_t)rem, div_k), kw = rem - kh * g.K;
      const int h = hb + kh * g.D, w = wb + kw * g.D;
      const bool ok = qv && j < g.J && (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
      rb[r] = xb[ok ? (int64_t)i * g.HW + h * g.W + w : 0];
      bm |= (uint32_t)ok << r;
    }
  };
  auto store = [&](float* buf) {
    float* As = buf;
    float* Bs = buf + TS::BK * TS::LDA;
#pragma unroll
    for (int r = 0; r < TS::A_PER_T; ++r)
      As[acol * TS::LDA + irow0 + ISTEP * r] = ((am >> r) & 1u) ? ra[r] : 0.f;
#pragma unroll
    for (int r = 0; r < TS::B_PER_T; ++r)
      Bs[(krow0 + KSTEP * r) * TS::LDB + pcol] = ((bm >> r) & 1u) ? rb[r] : 0.f;
  };

  Acc<TS> acc;
  acc.zero();
  gemm_mainloop<TS>(lds, 0, g.J, load, store, acc, wm, wn, wk, lane);
  reduce_wk<TS>(acc, lds, wm, wn, wk, lane);
  if (wk != 0) return;
#pragma unroll
  for (int aj = 0; aj < TS::RN; ++aj) {
    const int64_t qq = n0 + acc_n0<TS>(wn, aj) + acc_col(lane);
    if (qq >= g.Q) continue;
    const int b = (int)(qq / g.OHW), p = (int)(qq - (int64_t)b * g.OHW);
    float* zb = z + (int64_t)b * g.zs + p;
#pragma unroll
    for (int ai = 0; ai < TS::RM; ++ai)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = m0 + acc_m0<TS>(wm, ai) + acc_row(r, lane);
        if (o < g.OC) zb[(int64_t)o * g.OHW] = acc.v[ai][aj][r] + (bias ? bias[o] : 0.f);
      }
  }
}

// ---------------------------------------------------------------------------
// Layers with a short reduction (C*K*K <= 32, at most 32 output channels: a
// network's first layer on an image) are bound by writing z.  Each wave takes 32
// output pixels at a time as one 32 (o) x 32 (pixels) x 32 (j) matrix-core block
// (16 steps of v_mfma_f32_32x32x2_f32): the weights stay in registers for the
// whole kernel (lane l: W[l % 32][2s + l / 32]), each lane gathers the 16 taps
// 2s + l / 32 of pixel l % 32, and every accumulator row is one output channel's
// 32 consecutive pixels (coalesced stores).  Taps j >= J and channels o >= OC are
// zero operands.
// ---------------------------------------------------------------------------
constexpr int kSmallJ = 32, kSmallJOc = 32;

__global__ __launch_bounds__(kThreads) void conv_fwd_smallj(ConvGeom g, const float* __restrict__ x,
                                                           const float* __restrict__ wt,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ z, int64_t tiles) {
  // per tap j: its input-plane offset and its row / column shift under the window
  __shared__ int toff[kSmallJ], tdh[kSmallJ], tdw[kSmallJ];
  if (threadIdx.x < kSmallJ) {
    const int j = threadIdx.x, KK = g.K * g.K;
    const int i = j / KK, t = j - i * KK, kh = t / g.K, kw = t - kh * g.K;
    toff[j] = j < g.J ? i * g.HW : 0;
    // taps past J get a shift that is never inside the image: their operand is 0
    tdh[j] = j < g.J ? kh * g.D : -(1 << 28);
    tdw[j] = j < g.J ? kw * g.D : 0;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 31, kq = lane >> 5;
  float wa[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int j = 2 * s + kq;
    wa[s] = (m < g.OC && j < g.J) ? wt[m * g.J + j] : 0.f;
  }
  // the output channels this lane's accumulator rows hold, and their biases
  float bo[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int o = acc_row(r, lane);
    bo[r] = (bias && o < g.OC) ? bias[o] : 0.f;
  }
  for (int64_t tile = (int64_t)blockIdx.x * 4 + wave; tile < tiles;
       tile += (int64_t)gridDim.x * 4) {
    const int64_t q = tile * 32 + m;
    const bool qv = q < g.Q;
    int b = 0, r = 0, h0 = 0, w0 = 0;
    if (qv) {
      b = (int)(q / g.OHW);
      r = (int)(q - (int64_t)b * g.OHW);
      const int ho = r / g.OW, wo = r - ho * g.OW;
      h0 = ho * g.S - g.P;
      w0 = wo * g.S - g.P;
    }
    const float* xb = x + (int64_t)b * g.xs;
    float bv[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int j = 2 * s + kq;
      const int h = h0 + tdh[j], w = w0 + tdw[j];
      const bool ok = qv && (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
      bv[s] = ok ? xb[toff[j] + h * g.W + w] : 0.f;
    }
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(wa[s], bv[s], acc, 0, 0, 0);
    if (qv) {
      float* zb = z + (int64_t)b * g.zs + r;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int o = acc_row(i, lane);
        if (o < g.OC) zb[(int64_t)o * g.OHW] = acc[i] + bo[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The whole block forward of a layer with a short reduction (C*K*K <= 32, at most 32
// output channels) and batch normalisation, without ever storing z: its convolution
// costs 16 matrix-core steps per 32 pixels, far less than writing z and reading it
// back twice (statistics, then normalisation), so each of the two passes below
// computes z again from x, the way conv_fwd_smallj does.
//   fwd_first_stats: work-group blk takes pixels [blk*L, min(Q, (blk+1)*L)) of the
//     flattened (image, pixel) index for every output channel; each lane keeps, per
//     accumulator row (channel), the sums of d = z - K and d^2 with K the first z it
//     saw (as bnf_stats does), turns them into (count, mean, M2), and the 32 lanes of a
//     channel merge in a fixed butterfly, then the four waves in order, into
//     part[c][blk] = (mean, M2).
//   fwd_first_fold: per channel, one wave merges the work-groups' moments in double
//     (each lane a contiguous run in order, then a fixed butterfly): mean, biased var.
//   fwd_first_apply: z again, x_norm = (z - mean)/sqrt(var + eps), y = act(gamma x_norm
//     + beta) (bnf_apply's arithmetic), both stored; with fixed statistics only this.
// ---------------------------------------------------------------------------
struct FirstTaps {
  int off[kSmallJ], dh[kSmallJ], dw[kSmallJ];
};
// fwd_first_apply's activation as a template argument (the common ones compile to
// straight-line code); kActAnyFwd takes it from the run-time argument
constexpr int kActAnyFwd = -1;
// per tap j: its input-plane offset and its row / column shift under the window (taps
// past J get a shift that is never inside the image: their operand is 0)
__device__ __forceinline__ void first_taps(const ConvGeom& g, FirstTaps& t) {
  if (threadIdx.x < kSmallJ) {
    const int j = threadIdx.x, KK = g.K * g.K;
    const int i = j / KK, r = j - i * KK, kh = r / g.K, kw = r - kh * g.K;
    t.off[j] = j < g.J ? i * g.HW : 0;
    t.dh[j] = j < g.J ? kh * g.D : -(1 << 28);
    t.dw[j] = j < g.J ? kw * g.D : 0;
  }
}
// z of output pixel q (lane's column) for the 16 channels of this lane's accumulator
// rows: 16 steps of 32x32x2 over the taps 2s + lane / 32
__device__ __forceinline__ f32x16 first_z(const ConvGeom& g, const float* __restrict__ x,
                                          const FirstTaps& t, const float (&wa)[16], int64_t q,
                                          bool qv, int kq) {
  int b = 0, h0 = 0, w0 = 0;
  if (qv) {
    const uint32_t qq = (uint32_t)q;   // Q < 2^31 (checked on the host)
    b = (int)(qq / (uint32_t)g.OHW);
    const int r = (int)(qq - (uint32_t)b * (uint32_t)g.OHW);
    const int ho = r / g.OW, wo = r - ho * g.OW;
    h0 = ho * g.S - g.P;
    w0 = wo * g.S - g.P;
  }
  const float* xb = x + (int64_t)b * g.xs;
  float bv[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int j = 2 * s + kq;
    const int h = h0 + t.dh[j], w = w0 + t.dw[j];
    const bool ok = qv && (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
    bv[s] = ok ? xb[t.off[j] + h * g.W + w] : 0.f;
  }
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(wa[s], bv[s], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ void first_weights(const ConvGeom& g, const float* __restrict__ wt,
                                              float (&wa)[16], int lane) {
  const int m = lane & 31, kq = lane >> 5;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int j = 2 * s + kq;
    wa[s] = (m < g.OC && j < g.J) ? wt[m * g.J + j] : 0.f;
  }
}
__device__ __forceinline__ Moments shfl_moments(Moments m, int lane_mask) {
  return Moments{__shfl_xor(m.n, lane_mask), __shfl_xor(m.mean, lane_mask),
                 __shfl_xor(m.m2, lane_mask)};
}

__global__ __launch_bounds__(kThreads) void fwd_first_stats(ConvGeom g, const float* __restrict__ x,
                                                           const float* __restrict__ wt,
                                                           int64_t L, float2* __restrict__ part) {
  __shared__ FirstTaps taps;
  __shared__ Moments red[4][32];
  first_taps(g, taps);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, kq = lane >> 5;
  float wa[16];
  first_weights(g, wt, wa, lane);
  const int64_t q0 = (int64_t)blockIdx.x * L, q1 = min(g.Q, q0 + L);
  float K[16], s1[16], s2[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) K[r] = s1[r] = s2[r] = 0.f;
  int cnt = 0;
  for (int64_t t0 = q0 + 32 * wave; t0 < q1; t0 += 128) {
    const int64_t q = t0 + (lane & 31);
    const bool qv = q < q1;
    const f32x16 z = first_z(g, x, taps, wa, q, qv, kq);
    if (qv) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (cnt == 0) K[r] = z[r];
        const float d = z[r] - K[r];
        s1[r] += d;
        s2[r] += d * d;
      }
      ++cnt;
    }
  }
  // per channel row r: this lane's moments, then the 32 lanes holding the channel
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    Moments m{0.f, 0.f, 0.f};
    if (cnt > 0) {
      const float n = (float)cnt, mu = s1[r] / n;
      m = Moments{n, K[r] + mu, fmaxf(s2[r] - s1[r] * mu, 0.f)};
    }
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      const Moments o = shfl_moments(m, off);
      // the lower lane of each pair keeps (lower, upper); both end with the same value
      m = (lane & off) ? merge_moments(o, m) : merge_moments(m, o);
    }
    if ((lane & 31) == 0) red[wave][acc_row(r, lane)] = m;
  }
  __syncthreads();
  const int c = threadIdx.x;
  if (c < g.OC) {
    Moments m = red[0][c];
#pragma unroll
    for (int w = 1; w < 4; ++w) m = merge_moments(m, red[w][c]);
    part[(int64_t)c * gridDim.x + blockIdx.x] = make_float2(m.mean, m.m2);
  }
}

__global__ __launch_bounds__(64) void fwd_first_fold(const float2* __restrict__ part, int nblk,
                                                     int64_t L, int64_t Q, float* __restrict__ mean,
                                                     float* __restrict__ var) {
  const int c = blockIdx.x, lane = threadIdx.x;
  const int per = (nblk + 63) / 64, b0 = lane * per, b1 = min(nblk, b0 + per);
  double n = 0.0, mu = 0.0, m2 = 0.0;
  for (int b = b0; b < b1; ++b) {
    const double nb = (double)(min(Q, (int64_t)(b + 1) * L) - (int64_t)b * L);
    const float2 v = part[(int64_t)c * nblk + b];
    const double tot = n + nb, d = (double)v.x - mu;
    mu += d * nb / tot;
    m2 += (double)v.y + d * d * n * nb / tot;
    n = tot;
  }
  // lanes hold consecutive runs: merge (lower, upper) pairs in a fixed butterfly
  for (int off = 1; off < 64; off <<= 1) {
    const double on = __shfl_xor(n, off), omu = __shfl_xor(mu, off), om2 = __shfl_xor(m2, off);
    double an = n, amu = mu, am2 = m2, bn = on, bmu = omu, bm2 = om2;
    if (lane & off) { an = on; amu = omu; am2 = om2; bn = n; bmu = mu; bm2 = m2; }
    const double tot = an + bn;
    if (bn == 0.0) { n = an; mu = amu; m2 = am2; }
    else if (an == 0.0) { n = bn; mu = bmu; m2 = bm2; }
    else {
      const double d = bmu - amu;
      mu = amu + d * bn / tot;
      m2 = am2 + bm2 + d * d * an * bn / tot;
      n = tot;
    }
  }
  if (lane == 0) {
    mean[c] = (float)mu;
    var[c] = (float)(m2 / n);
  }
}

template <int ACT>
__global__ __launch_bounds__(kThreads, 4) void fwd_first_apply(
    ConvGeom g, const float* __restrict__ x, const float* __restrict__ wt,
    const float* __restrict__ mean, const float* __restrict__ var,
    const float* __restrict__ gamma, const float* __restrict__ beta, float eps, int act,
    float slope, float* __restrict__ xn, float* __restrict__ y, int64_t tiles) {
  __shared__ FirstTaps taps;
  __shared__ float prm[4][32];   // per channel: mean, 1/sqrt(var + eps), gamma, beta
  first_taps(g, taps);
  if (threadIdx.x < 32) {
    const int o = min((int)threadIdx.x, g.OC - 1);
    prm[0][threadIdx.x] = mean[o];
    prm[1][threadIdx.x] = 1.f / sqrtf(var[o] + eps);
    prm[2][threadIdx.x] = gamma[o];
    prm[3][threadIdx.x] = beta[o];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, kq = lane >> 5;
  float wa[16];
  first_weights(g, wt, wa, lane);
  const int a = ACT == kActAnyFwd ? act : ACT;
  for (int64_t tile = (int64_t)blockIdx.x * 4 + wave; tile < tiles;
       tile += (int64_t)gridDim.x * 4) {
    const int64_t q = tile * 32 + (lane & 31);
    const bool qv = q < g.Q;
    const f32x16 z = first_z(g, x, taps, wa, q, qv, kq);
    if (!qv) continue;
    const uint32_t b = (uint32_t)q / (uint32_t)g.OHW;
    const int64_t p = (int64_t)b * g.zs + ((uint32_t)q - b * (uint32_t)g.OHW);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int o = acc_row(r, lane);
      if (o >= g.OC) continue;
      const float xh = (z[r] - prm[0][o]) * prm[1][o];
      xn[p + (int64_t)o * g.OHW] = xh;
      y[p + (int64_t)o * g.OHW] = act_fwd(a, slope, prm[2][o] * xh + prm[3][o]);
    }
  }
}

// ---------------------------------------------------------------------------
// 3x3, pad-1, stride-2 forward (a downsampling layer: z of OH x OW from x of H x W)
// as a tile-direct implicit GEMM on the matrix cores.  A work-group owns 64 output
// channels (blockIdx.y) of one 16 x 16 output tile of one image and walks the input
// channels 4 at a time.  Per chunk the input patch under the tile (rows 2*h0-1 ..
// 2*h0+31, columns 2*w0-4 .. 2*w0+35 in 16-byte pieces; 0 off the image) is copied
// into LDS once by the LDS-DMA loads (padding pieces read a zero page), and the chunk's
// 64 x 36 weights go beside it as [channel, tap][o], copied in 16-byte pieces from the
// weights transposed to that order once per call (wtr[(i*9 + tap)*OCP + o], OCP = OC
// rounded up to 64, zero past OC: 64 consecutive o, where W's own order puts them C*9
// floats apart, a cache line per lane).  One 32x32x2 step takes two input channels at
// one tap (lanes 0-31 the first, 32-63 the second); each wave accumulates 2 (o) x 2
// (32 pixels = two tile rows) blocks over the 18 steps of a chunk.  A tap reads every
// other patch column (some bank conflicts: four LDS reads per 256 cycles of matrix
// work leave the LDS far from its limit).  Two LDS buffers, declared apart so that the
// compiler sees the copies into one never alias the matrix work's reads of the other:
// the next chunk's copies are in flight during this chunk's matrix work, one wait and
// one barrier per chunk.  A weight row (one (channel, tap) over 64 o) is 96 floats.
// Needs a width that is a multiple of 4 and 16-byte aligned x (checked at launch).
// ---------------------------------------------------------------------------
constexpr int kF2Tile = 16, kF2CC = 4, kF2PR = 33, kF2XP = 40, kF2CP = kF2PR * kF2XP, kF2WP = 96;
// 256-float copies (64 lanes x 16 bytes) per chunk: 21 of the patch, 14 of the weights
constexpr int kF2XN = (kF2CC * kF2CP + 255) / 256, kF2WN = (kF2CC * 9 * kF2WP + 255) / 256;
constexpr int kF2XFl = 256 * kF2XN, kF2WFl = 256 * kF2WN;   // floats per buffer

// Source of the zero padding of the copies (never written).
__device__ __align__(16) float g_fwd_zero[4];

template <bool BIAS>
__global__ __launch_bounds__(kThreads, 2) void conv_fwd3_s2(ConvGeom g, const float* __restrict__ x,
                                                           const float* __restrict__ wtr,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ z, int tiles_h,
                                                           int tiles_w) {
  __shared__ float X0[kF2XFl], W0[kF2WFl], X1[kF2XFl], W1[kF2WFl];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int tpi = tiles_h * tiles_w;
  const int b = blockIdx.x / tpi, tr = blockIdx.x - b * tpi;
  const int h0 = (tr / tiles_w) * kF2Tile, w0 = (tr % tiles_w) * kF2Tile;
  const int o0 = blockIdx.y * 64;
  const float* xb = x + (int64_t)b * g.xs;
  const int nch = (g.C + kF2CC - 1) / kF2CC;
  const int ocp = (g.OC + 63) / 64 * 64;   // row pitch of the transposed weights

  // offset inside a chunk of the 16-byte piece each of this lane's patch copies fetches
  // (-1: padding), the same for every chunk.  Piece u: channel u / 330, patch row
  // (u % 330) / 10, image columns 2*w0 - 4 + 4*(u % 10) .. + 3 (whole pieces: the width
  // is a multiple of 4).
  constexpr int XR = (kF2XN + 3) / 4;
  int xofs[XR];
#pragma unroll
  for (int r = 0; r < XR; ++r) {
    const int u = 64 * (wave + 4 * r) + lane;
    const int ch = u / (kF2CP / 4), rem = u - ch * (kF2CP / 4);
    const int row = rem / (kF2XP / 4), pc = rem - row * (kF2XP / 4);
    const int h = 2 * h0 - 1 + row, w = 2 * w0 - 4 + 4 * pc;
    const bool ok = ch < kF2CC && (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
    xofs[r] = ok ? (ch * g.H + h) * g.W + w : -1;
  }
  auto issue = [&](int c, float* Xl, float* Wl) {
    const int i0 = c * kF2CC;
    const float* xc = xb + (int64_t)i0 * g.HW;
#pragma unroll
    for (int r = 0; r < XR; ++r) {
      const int q = wave + 4 * r;
      int xo = xofs[r];
      asm volatile("" : "+v"(xo));   // keeps the 64-bit addresses from being hoisted
      const int ch = (64 * q + lane) / (kF2CP / 4);
      const float* src = xo >= 0 && i0 + ch < g.C ? xc + xo : g_fwd_zero;
      if (q < kF2XN) __builtin_amdgcn_global_load_lds(src, lds_ptr(Xl + 256 * q), 16, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < (kF2WN + 3) / 4; ++r) {
      const int q = wave + 4 * r;
      const int u = 4 * (64 * q + lane), kk = u / kF2WP, o = u - kk * kF2WP;
      const bool ok = kk < kF2CC * 9 && o < 64 && i0 + kk / 9 < g.C;
      const float* src = ok ? wtr + (int64_t)(i0 * 9 + kk) * ocp + o0 + o : g_fwd_zero;
      if (q < kF2WN) __builtin_amdgcn_global_load_lds(src, lds_ptr(Wl + 256 * q), 16, 0, 0);
    }
  };

  // this lane's operand offsets: A = W[o0 + 32 m + l32][(2 pc + hi, tap)], B = patch of
  // channel 2 pc + hi at pixel p = 32 nf + l32 (tile row p / 16, column p % 16) for the
  // wave's two pixel blocks nf = 2 wave, 2 wave + 1
  const int abase = hi * 9 * kF2WP + l32;
  int bbase[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int p = 32 * (2 * wave + f) + l32;
    bbase[f] = hi * kF2CP + 2 * (p >> 4) * kF2XP + 2 * (p & 15) + 3;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][f][r] = 0.f;

  // the operands of step k+1 are read from LDS while the matrix instructions of step k
  // issue (two register sets), so each step waits only for reads issued a step earlier
  auto compute = [&](const float* Xs, const float* Ws) {
    constexpr int NST = kF2CC / 2 * 9;
    float op[2][4];
    auto fetch = [&](int st, int sl) {
      const int pc = st / 9, t = st % 9, kh = t / 3, kw = t % 3;
      const int ao = (2 * pc * 9 + t) * kF2WP;
      const int bo = 2 * pc * kF2CP + kh * kF2XP + kw;
      op[sl][0] = Ws[abase + ao];
      op[sl][1] = Ws[abase + ao + 32];
      op[sl][2] = Xs[bbase[0] + bo];
      op[sl][3] = Xs[bbase[1] + bo];
    };
    fetch(0, 0);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int sl = st & 1;
      __builtin_amdgcn_sched_barrier(0);
      if (st + 1 < NST) fetch(st + 1, sl ^ 1);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(op[sl][0], op[sl][2], acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(op[sl][0], op[sl][3], acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(op[sl][1], op[sl][2], acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(op[sl][1], op[sl][3], acc[1][1], 0, 0, 0);
      if (st + 1 < NST) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // 4 LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                     // 4 MFMA
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // chunk c in buffer c & 1: wait for this wave's copies of it (nothing younger is in
  // flight), barrier (everyone's have landed and the other buffer's readers are done),
  // send the next chunk's copies into the other buffer, then the matrix work
  issue(0, X0, W0);
  for (int c = 0; c < nch; c += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (c + 1 < nch) issue(c + 1, X1, W1);
    compute(X0, W0);
    if (c + 1 >= nch) break;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (c + 2 < nch) issue(c + 2, X0, W0);
    compute(X1, W1);
  }

  // the biases added before the first store: no load is in flight among the stores
  // (a wait for a load there would also wait for every store before it)
  if constexpr (BIAS) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float bv = bias[min(o0 + 32 * m + acc_row(r, lane), g.OC - 1)];
        acc[m][0][r] += bv;
        acc[m][1][r] += bv;
        // the sums made here, not sunk into the conditional stores
        asm volatile("" : "+v"(acc[m][0][r]), "+v"(acc[m][1][r]));
      }
  }
  float* zb = z + (int64_t)b * g.zs;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int p = 32 * (2 * wave + f) + l32;
    const int ho = h0 + (p >> 4), wo = w0 + (p & 15);
    if (ho >= g.OH || wo >= g.OW) continue;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = o0 + 32 * m + acc_row(r, lane);
        if (o < g.OC) zb[(int64_t)o * g.OHW + ho * g.OW + wo] = acc[m][f][r];
      }
  }
}

// ---------------------------------------------------------------------------
// A plain stride-1 forward is the input gradient of another convolution:
//   z[n][o][h][w] = sum_{i,kh,kw} W[o][i][kh][kw] x[n][i][h + kh - P][w + kw - P]
//                 = sum_{i,kh,kw} W'[i][o][kh][kw] x[n][i][h + P' - kh][w + P' - kw]
// with W'[i][o][kh][kw] = W[o][i][K-1-kh][K-1-kw] and P' = K-1-P: the dX of a
// convolution whose input has OC channels of OH x OW and whose output has C
// channels of H x W (stride 1, pad P'), with dz := x and weights W'.  So the
// tiled input-gradient kernels compute the forward of the layers they cover.
// ---------------------------------------------------------------------------
static ConvGeom transposed_geom(const ConvGeom& g) {
  cbb_conv_desc d{};
  d.batch = g.N;
  d.in_c = g.OC;
  d.in_h = g.OH;
  d.in_w = g.OW;
  d.out_c = g.C;
  d.ksize = g.K;
  d.stride = 1;
  d.pad = g.K - 1 - g.P;
  return make_geom(d);
}

static bool forward_as_dx(const ConvGeom& g, bool has_bias) {
  return !has_bias && g.G == 1 && g.D == 1 && g.S == 1 && g.P <= g.K - 1 &&
         conv_dx_specialised(transposed_geom(g));
}

__global__ __launch_bounds__(kThreads) void flip_transpose_weights(const float* __restrict__ w,
                                                                   float* __restrict__ wt, int oc,
                                                                   int c, int k) {
  const int kk = k * k;
  const int64_t n = (int64_t)oc * c * kk;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * kThreads) {
    const int t = (int)(e % kk);
    const int64_t oi = e / kk;
    const int i = (int)(oi % c), o = (int)(oi / c);
    const int kh = t / k, kw = t - kh * k;
    wt[((int64_t)i * oc + o) * kk + (k - 1 - kh) * k + (k - 1 - kw)] = w[e];
  }
}

// wtr[(i*9 + tap)*ocp + o] = W[o][i][tap] (0 for o >= oc): the stride-2 kernel's
// weight order, ocp = oc rounded up to 64.
__global__ __launch_bounds__(kThreads) void transpose_weights3(const float* __restrict__ w,
                                                              float* __restrict__ wtr, int oc,
                                                              int ocp, int c) {
  const int64_t n = (int64_t)ocp * c * 9;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * kThreads) {
    const int64_t rem = e / ocp, o = e - rem * ocp;
    wtr[e] = o < oc ? w[o * c * 9 + rem] : 0.f;
  }
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

static bool forward_smallj(const ConvGeom& g) {
  return g.G == 1 && g.J <= kSmallJ && g.OC <= kSmallJOc;
}
static bool forward_s2(const ConvGeom& g) {
  return g.G == 1 && g.K == 3 && g.S == 2 && g.P == 1 && g.D == 1 && !forward_smallj(g);
}

// Pixels per work-group of fwd_first_stats: at most 768 work-groups (one round at three
// per CU), at least 512 pixels each, a multiple of 128 (one 32-pixel tile per wave per
// step).
static int64_t first_stats_len(const ConvGeom& g) {
  return std::max<int64_t>(512, ceil_div(ceil_div(g.Q, 768), 128) * 128);
}

bool conv_forward_first_fused(const ConvGeom& g, int bn) {
  return bn && forward_smallj(g) && g.Q < ((int64_t)1 << 31);   // 32-bit pixel division
}

// The fused block forward of a short-reduction layer with batch normalisation (bn 1:
// batch statistics, written to mean / var; 2: fixed, read).  ws: the moments,
// OC x ceil(Q / L) float2.
int launch_conv_block_forward_first(const ConvGeom& g, const float* x, const float* wt, int bn,
                                    float eps, int act, float slope, const float* gamma,
                                    const float* beta, float* mean, float* var, float* xn,
                                    float* y, float* ws, hipStream_t st) {
  if (bn == 1) {
    const int64_t L = first_stats_len(g);
    const int nblk = (int)ceil_div(g.Q, L);
    float2* part = reinterpret_cast<float2*>(ws);
    fwd_first_stats<<<(unsigned)nblk, kThreads, 0, st>>>(g, x, wt, L, part);
    int rc = check_launch("fwd_first_stats", st);
    if (rc) return rc;
    fwd_first_fold<<<(unsigned)g.OC, 64, 0, st>>>(part, nblk, L, g.Q, mean, var);
    rc = check_launch("fwd_first_fold", st);
    if (rc) return rc;
  }
  const int64_t tiles = ceil_div(g.Q, 32);
  const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(tiles, 4), 8192);
#define CBB_FIRST(A)                                                                        \
  fwd_first_apply<A><<<blocks, kThreads, 0, st>>>(g, x, wt, mean, var, gamma, beta, eps, act, \
                                                  slope, xn, y, tiles)
  if (act == CBB_ACT_LEAKY) CBB_FIRST(CBB_ACT_LEAKY);
  else if (act == CBB_ACT_LINEAR) CBB_FIRST(CBB_ACT_LINEAR);
  else if (act == CBB_ACT_RELU) CBB_FIRST(CBB_ACT_RELU);
  else CBB_FIRST(kActAnyFwd);
#undef CBB_FIRST
  return check_launch("fwd_first_apply", st);
}

// Scratch of the forward beyond the batch-norm partials: the flipped weights and
// the input-gradient kernel's own workspace when the forward runs as a dX; the
// transposed weights of the stride-2 kernel; the moments of the fused first-layer
// forward.
size_t conv_forward_workspace(const ConvGeom& g, bool has_bias) {
  size_t bytes = 0;
  if (forward_smallj(g))
    bytes = align_up((size_t)g.OC * ceil_div(g.Q, first_stats_len(g)) * sizeof(float2), 256);
  if (forward_s2(g))
    bytes = std::max(bytes, align_up((size_t)ceil_div(g.OC, 64) * 64 * g.C * 9 * sizeof(float), 256));
  if (forward_as_dx(g, has_bias)) {
    const size_t wbytes = align_up((size_t)g.OC * g.C * g.K * g.K * sizeof(float), 256);
    bytes = std::max(bytes, wbytes + conv_dx_workspace(transposed_geom(g)));
  }
  return bytes;
}

// z = conv(x, W) (+ bias).  g is the whole layer's geometry; a grouped layer runs
// all groups in one launch on the group geometry.
int launch_conv_forward(const ConvGeom& g, const float* x, const float* wt, const float* bias,
                        float* z, float* ws, hipStream_t st) {
  if (forward_as_dx(g, bias != nullptr)) {
    const ConvGeom t = transposed_geom(g);
    float* wflip = ws;
    float* ws2 = ws + align_up((size_t)g.OC * g.C * g.K * g.K * sizeof(float), 256) / sizeof(float);
    const int64_t n = (int64_t)g.OC * g.C * g.K * g.K;
    flip_transpose_weights<<<(unsigned)std::min<int64_t>(ceil_div(n, kThreads), 4096), kThreads, 0,
                             st>>>(wt, wflip, g.OC, g.C, g.K);
    const int rc = check_launch("flip_transpose_weights", st);
    if (rc) return rc;
    return launch_conv_dx(t, wflip, x, z, 0, ws2, st);
  }
  if (forward_smallj(g)) {
    const int64_t tiles = ceil_div(g.Q, 32);
    const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(tiles, 4), 8192);
    conv_fwd_smallj<<<blocks, kThreads, 0, st>>>(g, x, wt, bias, z, tiles);
    return check_launch("conv_fwd_smallj", st);
  }
  if (forward_s2(g) && g.W % 4 == 0 && aligned16(x)) {
    float* wtr = ws;
    const int ocp = (int)ceil_div(g.OC, 64) * 64;
    const int64_t n = (int64_t)ocp * g.C * 9;
    transpose_weights3<<<(unsigned)std::min<int64_t>(ceil_div(n, kThreads), 4096), kThreads, 0,
                         st>>>(wt, wtr, g.OC, ocp, g.C);
    const int rc = check_launch("transpose_weights3", st);
    if (rc) return rc;
    const int th = (int)ceil_div(g.OH, kF2Tile), tw = (int)ceil_div(g.OW, kF2Tile);
    const dim3 grid((unsigned)((int64_t)g.N * th * tw), (unsigned)ceil_div(g.OC, 64));
    if (bias)
      conv_fwd3_s2<true><<<grid, kThreads, 0, st>>>(g, x, wtr, bias, z, th, tw);
    else
      conv_fwd3_s2<false><<<grid, kThreads, 0, st>>>(g, x, wtr, bias, z, th, tw);
    return check_launch("conv_fwd3_s2", st);
  }
  ConvGeom s = g;
  s.C = g.C / g.G;
  s.OC = g.OC / g.G;
  s.J = s.C * g.K * g.K;
  const FastDiv dkk = make_fastdiv((uint32_t)(g.K * g.K)), dk = make_fastdiv((uint32_t)g.K);
  if (s.OC <= 32) {
    using TS = TileShape<1, 4, 1>;   // 32 output channels x 128 pixels
    const int tm = (int)ceil_div(s.OC, TS::BM);
    const dim3 grid((unsigned)(tm * ceil_div(g.Q, TS::BN)), (unsigned)g.G);
    conv_fwd_kernel<TS><<<grid, kThreads, 0, st>>>(s, x, wt, bias, z, tm, dkk, dk);
  } else {
    // 64 x 64 (measured faster than 64 x 128 on the 64-channel stride-2 stem layer)
    using TS = TileShape<2, 2, 1>;
    const int tm = (int)ceil_div(s.OC, TS::BM);
    const dim3 grid((unsigned)(tm * ceil_div(g.Q, TS::BN)), (unsigned)g.G);
    conv_fwd_kernel<TS><<<grid, kThreads, 0, st>>>(s, x, wt, bias, z, tm, dkk, dk);
  }
  return check_launch("conv_fwd_kernel", st);
}

}  // namespace cbb
