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

// Scratch of the forward beyond the batch-norm partials: the flipped weights and
// the input-gradient kernel's own workspace when the forward runs as a dX.
size_t conv_forward_workspace(const ConvGeom& g, bool has_bias) {
  if (!forward_as_dx(g, has_bias)) return 0;
  const size_t wbytes = align_up((size_t)g.OC * g.C * g.K * g.K * sizeof(float), 256);
  return wbytes + conv_dx_workspace(transposed_geom(g));
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
  if (g.G == 1 && g.J <= kSmallJ && g.OC <= kSmallJOc) {
    const int64_t tiles = ceil_div(g.Q, 32);
    const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(tiles, 4), 8192);
    conv_fwd_smallj<<<blocks, kThreads, 0, st>>>(g, x, wt, bias, z, tiles);
    return check_launch("conv_fwd_smallj", st);
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
