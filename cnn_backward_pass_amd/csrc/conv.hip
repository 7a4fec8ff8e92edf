// conv.hip -- weight and input gradients of a convolution as implicit GEMMs on
// the gfx950 fp32 matrix cores, with the im2col / col2im index maps applied
// while staging tiles into LDS (no column buffer is ever written).
//
// Pages: "YOLOv3 backpropagation: full-flow source analysis" (suzhouguqin.com),
// section 3.1 (backward_convolutional_layer: dW = delta x im2col(x)^T with
// beta = 1, dX = col2im(W^T x delta)) and section 3.2 (im2col_cpu/col2im_cpu
// index map, output size (size + 2 pad - k)/stride + 1).
#include <type_traits>

#include "cbb_internal.h"

namespace cbb {

// Kernels that form dz from delta, y and x_norm while staging it (DzSource) take
// the activation as a template argument: kFzOff = dz is read as it is, kFzAny =
// the activation is src.act at run time, else the activation itself.
constexpr int kFzOff = -2, kFzAny = -1;

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
                                                           int nsplits, int direct,
                                                           int64_t out_gstride) {
  // group blockIdx.y of a grouped convolution (g holds the group's channel counts)
  x += blockIdx.y * g.gx;
  dz += blockIdx.y * g.gz;
  out += blockIdx.y * out_gstride;
  __shared__ float lds[TS::LDS_FLOATS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % TS::WM, wn = (wave / TS::WM) % TS::WN, wk = wave / (TS::WM * TS::WN);
  // id = split * tiles + tile: the tiles of one split (same dz rows) are dispatched together
  const int tiles = gridDim.x / nsplits;
  const int lid = blockIdx.x;
  const int split = lid / tiles, tile = lid - split * tiles;
  const int m0 = (tile / tiles_n) * TS::BM, n0 = (tile % tiles_n) * TS::BN;
  const int64_t kbeg = (int64_t)split * k_chunk;
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
      boff[r] = i * g.HW + (kh * g.W + kw) * g.D;
      bkh[r] = kh * g.D;
      bkw[r] = kw * g.D;
    } else {  // column beyond J: force the bounds test to fail
      boff[r] = 0;
      bkh[r] = -(1 << 28);
      bkw[r] = 0;
    }
  }

  // Loads go to registers as they are; the zero padding is applied when they
  // are stored to LDS, so no loaded value is consumed before the next tile and
  // the loads stay in flight during the matrix-core work.
  static_assert(TS::A_PER_T <= 32 && TS::B_PER_T <= 32, "one mask bit per staged element");
  float ra[TS::A_PER_T], rb[TS::B_PER_T];
  uint32_t am = 0, bm = 0;
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
    // Out-of-range elements load from a clamped (valid) address: no divergent
    // branches around the loads.
    const float* db = dz + (int64_t)b * g.zs + rem;
    am = 0;
    bm = 0;
#pragma unroll
    for (int r = 0; r < TS::A_PER_T; ++r) {
      const int o = m0 + rbase + RSTEP * r;
      const bool ok = qv && o < g.OC;
      ra[r] = db[(int64_t)(ok ? o : 0) * g.OHW];
      am |= (uint32_t)ok << r;
    }
    // x index of (n, i, hb + kh, wb + kw) = image base + boff + hb*W + wb
    const float* xb = x + (int64_t)b * g.xs;
    const int pbase = hb * g.W + wb;
#pragma unroll
    for (int r = 0; r < TS::B_PER_T; ++r) {
      const int h = hb + bkh[r], w = wb + bkw[r];
      const bool ok = qv && (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
      rb[r] = xb[ok ? boff[r] + pbase : 0];
      bm |= (uint32_t)ok << r;
    }
  };
  auto store = [&](float* buf) {
    float* As = buf;
    float* Bs = buf + TS::BK * TS::LDA;
#pragma unroll
    for (int r = 0; r < TS::A_PER_T; ++r)
      As[qi * TS::LDA + rbase + RSTEP * r] = ((am >> r) & 1u) ? ra[r] : 0.f;
#pragma unroll
    for (int r = 0; r < TS::B_PER_T; ++r)
      Bs[qi * TS::LDB + rbase + RSTEP * r] = ((bm >> r) & 1u) ? rb[r] : 0.f;
  };

  Acc<TS> acc;
  acc.zero();
  gemm_mainloop<TS>(lds, kbeg, kend, load, store, acc, wm, wn, wk, lane);
  reduce_wk<TS>(acc, lds, wm, wn, wk, lane);
  if (wk == 0) {
    float* dst = direct ? out : out + (int64_t)split * g.OC * g.J;
#pragma unroll
    for (int ai = 0; ai < TS::RM; ++ai)
#pragma unroll
      for (int aj = 0; aj < TS::RN; ++aj) {
        const int j = n0 + acc_n0<TS>(wn, aj) + acc_col(lane);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = m0 + acc_m0<TS>(wm, ai) + acc_row(r, lane);
          if (o < g.OC && j < g.J) {
            const int64_t e = (int64_t)o * g.J + j;
            if (direct)
              dst[e] += acc.v[ai][aj][r];
            else
              dst[e] = acc.v[ai][aj][r];
          }
        }
      }
  }
}

// Ordered sum of the dW split partials.  Level 1 (only when there are many
// splits): work-group (e-block, g) sums splits [g*SG, (g+1)*SG) of 256
// consecutive elements into part2[g][e].  Level 2: dw[e] += sum over g (or over
// the splits directly) in index order.  Every output element is summed by one
// thread in a fixed order, so the result does not depend on scheduling.

// part[s0*mn + e] + ... + part[(s1-1)*mn + e] for W = 1 or 4 consecutive elements
// (one float or one 16-byte piece per split), added in index order; the loads go
// out eight at a time (clamped to the last split, so every address is valid; the
// extra values are not added).
typedef float rf4 __attribute__((ext_vector_type(4)));
constexpr int64_t kRedVecMin = int64_t(1) << 20;   // elements: 16-byte form from here on
template <int W>
using RedVec = typename std::conditional<W == 4, rf4, float>::type;

template <int W>
__device__ __forceinline__ RedVec<W> vsum_in_order(const float* __restrict__ part, int s0, int s1,
                                                   int64_t mn, int64_t e) {
  using V = RedVec<W>;
  auto ld = [&](int k) { return *reinterpret_cast<const V*>(part + (int64_t)k * mn + e); };
  V acc = ld(s0);
  for (int k = s0 + 1; k < s1; k += 8) {
    V v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ld(min(k + u, s1 - 1));
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k + u < s1) acc += v[u];
  }
  return acc;
}

template <int W>
__global__ __launch_bounds__(kThreads) void dw_reduce_l1(const float* __restrict__ part,
                                                         float* __restrict__ part2, int splits,
                                                         int64_t mn, int64_t region) {
  part += blockIdx.z * region;    // grouped convolution: one partial region per group
  part2 += blockIdx.z * region;
  const int64_t e = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * W;
  if (e >= mn) return;
  const int s0 = blockIdx.y * kReduceGroup, s1 = min(splits, s0 + kReduceGroup);
  *reinterpret_cast<RedVec<W>*>(part2 + (int64_t)blockIdx.y * mn + e) =
      vsum_in_order<W>(part, s0, s1, mn, e);
}

// Partials in dW's own [o][i][tap] order: dw[e] += their ordered sum.
template <int W>
__global__ __launch_bounds__(kThreads) void dw_reduce_l2(float* __restrict__ dw,
                                                         const float* __restrict__ part, int n,
                                                         int64_t mn, int64_t region) {
  part += blockIdx.z * region;    // grouped convolution: group blockIdx.z's partials
  dw += blockIdx.z * mn;          // and its dW block
  const int64_t e = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * W;
  if (e >= mn) return;
  RedVec<W>* d = reinterpret_cast<RedVec<W>*>(dw + e);
  *d += vsum_in_order<W>(part, 0, n, mn, e);
}

// Tap-major partials [tap][o][i] (9 taps, oc x c per tap), which the row-streaming
// kernel writes so that its stores are contiguous: work-group (i block, o) sums
// taps x 64 input channels with coalesced reads (thread = (tap, i)), regroups them
// in LDS and adds them into dW's [o][i][tap] order as one contiguous run.
constexpr int kTapRedThreads = 9 * 64;
__global__ __launch_bounds__(kTapRedThreads) void dw_reduce_tap(float* __restrict__ dw,
                                                               const float* __restrict__ part,
                                                               int n, int64_t mn, int oc, int c,
                                                               int64_t region) {
  part += blockIdx.z * region;
  dw += blockIdx.z * mn;
  __shared__ float tile[kTapRedThreads];
  const int tid = threadIdx.x, tap = tid >> 6, il = tid & 63;
  const int o = blockIdx.y, i0 = blockIdx.x * 64, ni = min(64, c - i0);
  if (il < ni)
    tile[il * 9 + tap] =
        vsum_in_order<1>(part, 0, n, mn, ((int64_t)tap * oc + o) * c + i0 + il);
  __syncthreads();
  if (tid < 9 * ni) dw[((int64_t)o * c + i0) * 9 + tid] += tile[tid];
}

// ---------------------------------------------------------------------------
// Weight gradient of a 3x3, pad-1 convolution at stride 1 or 2, row-streaming
// tile-direct form (same sum as conv_dw_kernel, no im2col gather).
//
// A work-group owns a 64 (o) x 32 (i) block of dW for all nine taps and a run
// of consecutive output rows over a strip of TC output columns of one image.
// The three input rows under the current output row stay in an LDS ring
// (input row h in slot h mod 3), so each input row is fetched once per run:
// per output row only the S new input rows and the dz row are loaded, into
// registers, while the matrix cores work on the previous row.  The reduction
// index runs over output positions, two per 32x32x2 step: lane l of a step
// takes column 2s + l/32 of the row, dz[o = l%32] as the A operand and
// x[i = l%32] under tap (kh, kw) as the B operand; the tap shifts are constant
// LDS offsets.  Twelve waves -- (o half) x (tap row kh) x (half of the row's
// steps) -- each hold the three accumulators of their taps; twelve waves put
// the same number of waves on each of the CU's four SIMDs (a six-wave group
// measured 15-20% slower).  The two step halves are summed through LDS at the
// end; each work-group writes its partial dW block (tap-major, contiguous
// stores) for the ordered split reduction, or adds into dW when it is the
// only split.
// ---------------------------------------------------------------------------
constexpr int kDw3Threads = 768;

template <int S, int TC>
struct Dw3RowCfg {
  static constexpr int KS = TC / 2;            // 32x32x2 steps per output row
  static constexpr int KH = (KS + 1) / 2;      // steps per half
  static constexpr int XC = S * (TC - 1) + 3;  // input columns under TC output columns
  // input column j of a channel sits at LDS column X0 + j: the three columns before
  // it take the head of the first 16-byte piece, so whole pieces are stored (the
  // XP pieces of a row cover LDS columns 0 .. 4 XP - 1, all inside the pitch)
  static constexpr int X0 = 3;
  static constexpr int XP = (XC + 6) / 4;
  static constexpr int CS = ((XC + X0) > 4 * XP ? XC + X0 : 4 * XP) | 1;   // channel pitch (odd)
  static constexpr int SLOT = 32 * CS;
  static constexpr int NSLOT = 3 + S;          // ring: the three rows in use + the S arriving
  static constexpr int OS = TC + 1;            // dz row pitch per output channel (odd)
  static constexpr int Z0 = NSLOT * SLOT;      // two dz row buffers after the slots
  static constexpr int ZB = 64 * OS;
  static constexpr int RED = 6 * 3 * 16 * 64;  // step-half exchange: 6 waves x 3 accumulators
  static constexpr int LDS_FLOATS = (Z0 + 2 * ZB) > RED ? (Z0 + 2 * ZB) : RED;
  static constexpr bool FITS = LDS_FLOATS * 4 <= 160 * 1024;
  static constexpr int XNEW = S * 32 * XC;     // floats of the S input rows fetched per row
  static constexpr int XPT = (XNEW + kDw3Threads - 1) / kDw3Threads;
  static constexpr int ZNEW = 64 * TC;
  static constexpr int ZPT = (ZNEW + kDw3Threads - 1) / kDw3Threads;
  static_assert(TC % 2 == 0 && (S == 1 || S == 2), "even strip, stride 1 or 2");
};

// V4: 16-byte loads (the host checks that W and OW are multiples of 4, TC too,
// and that x and dz are 16-byte aligned); x pieces start three columns before
// LDS column 0 and the extra columns are dropped at the LDS store.
// FZ != kFzOff (16-byte path only): the dz argument is delta; dz is formed from
// delta, y and x_norm with the per-channel map in src while it is staged, and the
// work-groups of the first input-channel block also write it to dzout (each dz
// element is staged by exactly one work-group per input-channel block), so the
// input-gradient kernel can read it afterwards.
template <int S, int TC, bool V4, int FZ = kFzOff>
__global__ __launch_bounds__(kDw3Threads, 1) void conv_dw3_rows(
    ConvGeom g, const float* __restrict__ x, const float* __restrict__ dz, float* __restrict__ out,
    int strips, int rchunks, int rlen, int direct, DzSource src, float* __restrict__ dzout,
    int64_t out_gstride) {
  using Cf = Dw3RowCfg<S, TC>;
  // group blockIdx.y of a grouped convolution (g holds the group's channel counts and
  // the whole tensors' image strides; dz is formed only on plain layers)
  x += blockIdx.y * g.gx;
  dz += blockIdx.y * g.gz;
  out += blockIdx.y * out_gstride;
  constexpr int NT = kDw3Threads;
  __shared__ float lds[Cf::LDS_FLOATS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int oh = wave & 1, kh = (wave >> 1) % 3, kq = wave / 6;
  const int cblocks = g.C >> 5, nblk = (g.OC >> 6) * cblocks;
  // XCD-aware order: consecutive logical indices run on one XCD (one L2), and they
  // go (o, i) block first, then strip: the blocks that stage the same input and dz
  // rows, and the strips whose row pieces share cache lines, hit one L2.
  const int bid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int blk = bid % nblk, t0 = bid / nblk;
  const int strip = t0 % strips, t1 = t0 / strips;
  const int rc = t1 % rchunks, n = t1 / rchunks;
  const int split = (n * rchunks + rc) * strips + strip;
  const int ob = blk / cblocks, cb = blk - ob * cblocks;
  const int r0 = rc * rlen, r1 = min(g.OH, r0 + rlen);  // non-empty by construction
  const int oc0 = strip * TC;       // first output column of the strip
  const int ic0 = oc0 * S - 1;      // input column held in LDS column 0
  const float* xb = x + (int64_t)n * g.xs + (int64_t)cb * 32 * g.HW;
  const float* zb = dz + (int64_t)n * g.zs + (int64_t)ob * 64 * g.OHW;
  constexpr bool fz = FZ != kFzOff, fz_y = fz && FZ != CBB_ACT_LINEAR;
  static_assert(!fz || V4, "dz is formed on the 16-byte path only");
  const int64_t zoff = ((int64_t)n * g.OC + ob * 64) * g.OHW;
  const float* yb = fz_y ? src.y + zoff : zb;
  const float* nb = fz && src.xn ? src.xn + zoff : zb;   // without x_norm: c = 0
  float* dzw = fz && cb == 0 ? dzout + zoff : nullptr;

  // Ring rows fetched with output row q: h = S*q + 2 - S + rr, rr < S.  The
  // loads go to registers as they are (positions off the image read a clamped
  // valid address) and the zero padding is applied when they are written to
  // LDS, so nothing consumes a loaded value before the next row: the loads
  // stay in flight during the matrix-core work.
  static_assert(Cf::XPT <= 32 && Cf::ZPT <= 32, "one mask bit per fetched element");
  static_assert(!V4 || TC % 4 == 0, "16-byte loads need a strip width multiple of 4");
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int XV = Cf::XP;   // 16-byte pieces per input row (columns -3 ..)
  constexpr int XNEW4 = S * 32 * XV, XPT4 = (XNEW4 + NT - 1) / NT;
  constexpr int ZV = TC / 4, ZNEW4 = 64 * ZV, ZPT4 = (ZNEW4 + NT - 1) / NT;
  float px[V4 ? 1 : Cf::XPT], pz[V4 ? 1 : Cf::ZPT];
  f4 px4[V4 ? XPT4 : 1], pz4[V4 ? ZPT4 : 1];
  f4 py4[fz ? ZPT4 : 1], pn4[fz ? ZPT4 : 1];
  uint32_t xm = 0, zm = 0;
  // the map of the channels this thread stages (fixed over the rows)
  float ka[fz ? ZPT4 : 1], kb[fz ? ZPT4 : 1], kc[fz ? ZPT4 : 1];
  if constexpr (fz) {
#pragma unroll
    for (int i = 0; i < ZPT4; ++i) {
      const int e = tid + i * NT;
      const int o = ob * 64 + min(e / ZV, 63);
      ka[i] = src.coef[o];
      kb[i] = src.coef[g.OC + o];
      kc[i] = src.coef[2 * g.OC + o];
    }
  }
  // Input rows (x) and the dz row are fetched and committed separately, so each
  // part can go between matrix-core steps of the previous row.
  auto fetch_x = [&](int q) {
    const int hb = S * q + 2 - S;
    xm = 0;
    if constexpr (V4) {
#pragma unroll
      for (int i = 0; i < XPT4; ++i) {
        const int e = tid + i * NT;
        const int rr = e / (32 * XV), rem = e - rr * (32 * XV);
        const int c = rem / XV, v = rem - c * XV;
        const int h = hb + rr, w = ic0 - 3 + 4 * v;
        const bool ok = e < XNEW4 && (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
        px4[i] = *(const f4*)(xb + (ok ? c * g.HW + h * g.W + w : 0));
        xm |= (uint32_t)ok << i;
      }
    } else {
#pragma unroll
      for (int i = 0; i < Cf::XPT; ++i) {
        const int e = tid + i * NT;
        const int rr = e / (32 * Cf::XC), rem = e - rr * (32 * Cf::XC);
        const int c = rem / Cf::XC, j = rem - c * Cf::XC;
        const int h = hb + rr, w = ic0 + j;
        const bool ok =
            e < Cf::XNEW && (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
        px[i] = xb[ok ? c * g.HW + h * g.W + w : 0];
        xm |= (uint32_t)ok << i;
      }
    }
  };
  auto fetch_z = [&](int q) {
    zm = 0;
    if constexpr (V4) {
#pragma unroll
      for (int i = 0; i < ZPT4; ++i) {
        const int e = tid + i * NT;
        const int o = e / ZV, v = e - o * ZV;
        const bool ok = e < ZNEW4 && oc0 + 4 * v < g.OW;
        const int zo = ok ? o * g.OHW + q * g.OW + oc0 + 4 * v : 0;
        pz4[i] = *(const f4*)(zb + zo);
        if constexpr (fz_y) py4[i] = *(const f4*)(yb + zo);
        if constexpr (fz) pn4[i] = *(const f4*)(nb + zo);
        zm |= (uint32_t)ok << i;
      }
    } else {
#pragma unroll
      for (int i = 0; i < Cf::ZPT; ++i) {
        const int e = tid + i * NT;
        const int o = e / TC, j = e - o * TC;
        const bool ok = e < Cf::ZNEW && oc0 + j < g.OW;
        pz[i] = zb[ok ? o * g.OHW + q * g.OW + oc0 + j : 0];
        zm |= (uint32_t)ok << i;
      }
    }
  };
  auto commit_x = [&](int q) {
    const int hb = S * q + 2 - S;
    if constexpr (V4) {
#pragma unroll
      for (int i = 0; i < XPT4; ++i) {
        const int e = tid + i * NT;
        const int rr = e / (32 * XV), rem = e - rr * (32 * XV);
        const int c = rem / XV, v = rem - c * XV;
        if (e < XNEW4) {
          // piece v holds input columns 4v - 3 .. 4v (LDS columns 4v .. 4v + 3, all
          // inside the channel's pitch; the ones outside 0 .. XC-1 are never read)
          float* d = lds + ((hb + rr + Cf::NSLOT) % Cf::NSLOT) * Cf::SLOT + c * Cf::CS + 4 * v;
          const bool ok = (xm >> i) & 1u;
#pragma unroll
          for (int u = 0; u < 4; ++u) d[u] = ok ? px4[i][u] : 0.f;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < Cf::XPT; ++i) {
        const int e = tid + i * NT;
        const int rr = e / (32 * Cf::XC), rem = e - rr * (32 * Cf::XC);
        const int c = rem / Cf::XC, j = rem - c * Cf::XC;
        if (e < Cf::XNEW)
          lds[((hb + rr + Cf::NSLOT) % Cf::NSLOT) * Cf::SLOT + c * Cf::CS + Cf::X0 + j] =
              ((xm >> i) & 1u) ? px[i] : 0.f;
      }
    }
  };
  auto commit_z = [&](int q) {
    if constexpr (V4) {
#pragma unroll
      for (int i = 0; i < ZPT4; ++i) {
        const int e = tid + i * NT;
        const int o = e / ZV, v = e - o * ZV;
        if (e < ZNEW4) {
          float* d = lds + Cf::Z0 + (q & 1) * Cf::ZB + o * Cf::OS + 4 * v;
          const bool ok = (zm >> i) & 1u;
          f4 val = pz4[i];
          if constexpr (fz) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              float gv = val[u];
              if constexpr (fz_y) gv *= act_grad(FZ == kFzAny ? src.act : FZ, src.slope, py4[i][u]);
              val[u] = ka[i] * gv + kb[i] + kc[i] * pn4[i][u];
            }
            if (dzw && ok) *(f4*)(dzw + o * g.OHW + q * g.OW + oc0 + 4 * v) = val;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) d[u] = ok ? val[u] : 0.f;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < Cf::ZPT; ++i) {
        const int e = tid + i * NT;
        const int o = e / TC, j = e - o * TC;
        if (e < Cf::ZNEW)
          lds[Cf::Z0 + (q & 1) * Cf::ZB + o * Cf::OS + j] = ((zm >> i) & 1u) ? pz[i] : 0.f;
      }
    }
  };

  // The 3 - S ring rows of the first output row that no fetch covers.
  for (int e = tid; e < (3 - S) * 32 * Cf::XC; e += NT) {
    const int rr = e / (32 * Cf::XC), rem = e - rr * (32 * Cf::XC);
    const int c = rem / Cf::XC, j = rem - c * Cf::XC;
    const int h = S * r0 - 1 + rr, w = ic0 + j;
    const bool ok = (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
    const float v = xb[ok ? c * g.HW + h * g.W + w : 0];
    lds[((h + Cf::NSLOT) % Cf::NSLOT) * Cf::SLOT + c * Cf::CS + Cf::X0 + j] = ok ? v : 0.f;
  }
  fetch_x(r0);
  fetch_z(r0);
  commit_x(r0);
  commit_z(r0);
  __syncthreads();
  if (r0 + 1 < r1) {
    fetch_x(r0 + 1);
    fetch_z(r0 + 1);
  }

  f32x16 acc[3];
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;

  // this wave's half of the row: steps [kq*KH, min(KS, kq*KH + KH))
  const int abase0 = Cf::Z0 + (32 * oh + (lane & 31)) * Cf::OS + (lane >> 5) + 2 * Cf::KH * kq;
  const int bbase = (lane & 31) * Cf::CS + Cf::X0 + S * (lane >> 5) + 2 * S * Cf::KH * kq;
  // One barrier per row: the rows and the dz buffer that arrive for row r+1 go
  // to slots (buffer) that row r does not read.  When dz is formed here (three
  // tensors' rows to stage and transform per row), each wave stages its part of
  // row r+1 between its own matrix-core steps on row r (input rows after the
  // second step, the dz row half way) and sends the loads for row r+2 as soon as
  // the registers they land in are free: stem conv2 (16x32x416x416 -> 64, s2)
  // 321 -> 284 us.  With a stored dz the staging is light and it goes after the
  // row's matrix work (interleaved it measured 4-6% slower on the 52x52 and
  // 26x26 layers).  (The run-time activation switch on 104-column strips would
  // not fit the registers interleaved.)
  constexpr bool kInter = fz && (FZ != kFzAny || TC <= 64);
  constexpr int kStepX = Cf::KH > 2 ? 1 : 0, kStepZ = Cf::KH > 4 ? Cf::KH / 2 : Cf::KH - 1;
  for (int r = r0; r < r1; ++r) {
    // input row S*r - 1 + kh sits in slot (S*r - 1 + kh) mod NSLOT
    const int bs = ((S * r + kh - 1 + Cf::NSLOT) % Cf::NSLOT) * Cf::SLOT + bbase;
    const int abase = abase0 + (r & 1) * Cf::ZB;
    const bool next = r + 1 < r1, next2 = r + 2 < r1;
#pragma unroll
    for (int sp = 0; sp < Cf::KH; ++sp) {
      if (Cf::KS % 2 == 0 || kq == 0 || sp < Cf::KS / 2) {
        const float a = lds[abase + 2 * sp];
        float b[3];
#pragma unroll
        for (int kw = 0; kw < 3; ++kw) b[kw] = lds[bs + 2 * S * sp + kw];
#pragma unroll
        for (int kw = 0; kw < 3; ++kw)
          acc[kw] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b[kw], acc[kw], 0, 0, 0);
      }
      if (kInter && sp == kStepX && next) {
        commit_x(r + 1);
        if (next2) fetch_x(r + 2);
      }
      if (kInter && sp == kStepZ && next) {
        commit_z(r + 1);
        if (next2) fetch_z(r + 2);
      }
    }
    if (!kInter && next) {
      commit_x(r + 1);
      commit_z(r + 1);
      if (next2) {
        fetch_x(r + 2);
        fetch_z(r + 2);
      }
    }
    __syncthreads();
  }

  // Sum the step halves: waves kq = 1 hand their accumulators over through LDS.
  __syncthreads();
  if (kq == 1) {
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) lds[(((wave - 6) * 3 + t) * 16 + r) * 64 + lane] = acc[t][r];
  }
  __syncthreads();
  if (kq == 1) return;
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] += lds[((wave * 3 + t) * 16 + r) * 64 + lane];

  // the only split adds into dW ([o][i][tap]); partials are tap-major [tap][o][i]
  // (contiguous stores), mapped back by the reduction
  const int i = cb * 32 + (lane & 31);
#pragma unroll
  for (int kw = 0; kw < 3; ++kw)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int o = ob * 64 + 32 * oh + acc_row(r, lane);
      const int t = kh * 3 + kw;
      if (direct)
        out[(int64_t)o * g.J + i * 9 + t] += acc[kw][r];
      else
        out[(int64_t)split * g.OC * g.J + ((int64_t)t * g.OC + o) * g.C + i] = acc[kw][r];
    }
}

// ---------------------------------------------------------------------------
// Input gradient, gather form of col2im(W^T x delta).  For stride s the input
// pixels split into s*s phases (h mod s, w mod s); inside a phase every pixel
// receives the same set of taps kh = rh + s*th (rh = (ph + p) mod s), and the
// output row it reads is ho = (h + p - kh)/s = hh + bh - th with h = ph + s*hh,
// bh = (ph + p - rh)/s.  Each phase is a dense GEMM
//   dx[i][pix] = sum_kk A[i][kk] * B[kk][pix],   kk = t*OCP + o (tap-major),
//   A[i][kk] = W[o][i][kh][kw],  B[kk][pix] = dz[n][o][ho][wo] (0 off the map),
// so no matrix-core work is spent on the stride's empty taps.  OCP is C_out
// rounded up to the K tile (rows o >= C_out are zero), so a K tile never
// straddles two taps: the tap and the tile's first channel are uniform over
// the work-group and the per-element index math is an add.
// Grid: x = pixel tiles, y = channel tiles x K splits, z = phase.  With one
// split the result goes to dx (overwrite or add); with several, each split
// writes its partial at the pixel's dx position in ws[split] and
// dx_splitk_reduce adds them up in order.
// ---------------------------------------------------------------------------
template <class TS>
__global__ __launch_bounds__(kThreads) void conv_dx_kernel(ConvGeom g, const float* __restrict__ wt,
                                                           const float* __restrict__ dz,
                                                           float* __restrict__ dx,
                                                           float* __restrict__ ws, int ctiles,
                                                           int ksplits, int pixtiles,
                                                           int accumulate) {
  static_assert(kThreads % TS::BN == 0 && kThreads % TS::BK == 0, "thread/tile mapping");
  // group blockIdx.y of a grouped convolution (g holds the group's channel counts)
  wt += blockIdx.y * g.gw;
  dz += blockIdx.y * g.gz;
  dx += blockIdx.y * g.gx;
  if (ws) ws += blockIdx.y * g.gx;
  __shared__ float lds[TS::LDS_FLOATS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % TS::WM, wn = (wave / TS::WM) % TS::WN, wk = wave / (TS::WM * TS::WN);

  // id = ((phase * pixtiles + pixtile) * ksplits + split) * ctiles + ctile: the channel
  // tiles of one pixel tile read the same dz and are dispatched together.
  const int S = g.S;
  int lid = blockIdx.x;
  const int ctile = lid % ctiles;
  lid /= ctiles;
  const int split = lid % ksplits;
  lid /= ksplits;
  const int pixtile = lid % pixtiles, phase = lid / pixtiles;
  const int ph = phase / S, pw = phase % S;
  const int HH = (g.H - ph + S - 1) / S, WW = (g.W - pw + S - 1) / S;
  const int npix = g.N * HH * WW;
  const int n0 = pixtile * TS::BN;
  if (n0 >= npix) return;  // this phase has fewer pixels than the grid covers
  const int m0 = ctile * TS::BM;
  // Taps that reach this phase: kh with (ph + P - kh*D) divisible by S, i.e.
  // kh = rh, rh + SK, rh + 2 SK, ... with SK = S / gcd(D, S); along them the
  // output row moves down by DS = D / gcd(D, S) (S and 1 when D = 1).
  int gcd = S, dd = g.D;
  while (dd) {
    const int t = gcd % dd;
    gcd = dd;
    dd = t;
  }
  const int SK = S / gcd, DS = g.D / gcd;
  int rh = g.K, rw = g.K;
  for (int k = g.K - 1; k >= 0; --k) {
    if ((ph + g.P - k * g.D) % S == 0) rh = k;
    if ((pw + g.P - k * g.D) % S == 0) rw = k;
  }
  const int nkh = rh < g.K ? (g.K - rh + SK - 1) / SK : 0;
  const int nkw = rw < g.K ? (g.K - rw + SK - 1) / SK : 0;
  const int bh = (ph + g.P - rh * g.D) / S, bw = (pw + g.P - rw * g.D) / S;
  const int OCP = (g.OC + TS::BK - 1) / TS::BK * TS::BK;
  const int KT = OCP * nkh * nkw;
  const int kchunk = ((KT + ksplits - 1) / ksplits + TS::BK - 1) / TS::BK * TS::BK;
  const int kbeg = split * kchunk, kend = min(KT, kbeg + kchunk);

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
  const float* dzb = dz + (int64_t)pb * g.zs;
  const int hob = phh + bh, wob = pww + bw;

  // A: this thread stages K column acol for channel rows m0 + irow0 + ISTEP*r.
  constexpr int ISTEP = kThreads / TS::BK;
  const int acol = tid % TS::BK, irow0 = tid / TS::BK;
  const int KK = g.K * g.K;

  // Out-of-range elements load from a clamped (valid) address (no divergent
  // branches around the loads); the zero padding is applied at the LDS store,
  // so the loads stay in flight during the matrix-core work.
  static_assert(TS::A_PER_T <= 32 && TS::B_PER_T <= 32, "one mask bit per staged element");
  float ra[TS::A_PER_T], rb[TS::B_PER_T];
  uint32_t am = 0, bm = 0;
  auto load = [&](int k0) {
    const int t = k0 / OCP, o0 = k0 - t * OCP;  // uniform over the work-group
    const int th = t / nkw, tw = t - th * nkw;
    const int kh = rh + SK * th, kw = rw + SK * tw;
    {  // A = weights
      const int o = o0 + acol;
      const bool ov = o < g.OC;
      const float* wp = wt + ((int64_t)(ov ? o : 0) * g.C) * KK + kh * g.K + kw;
      am = 0;
#pragma unroll
      for (int r = 0; r < TS::A_PER_T; ++r) {
        const int i = m0 + irow0 + ISTEP * r;
        const bool ok = ov && i < g.C;
        ra[r] = wp[(int64_t)(ok ? i : 0) * KK];
        am |= (uint32_t)ok << r;
      }
    }
    {  // B = deltas
      const int ho = hob - th * DS, wo = wob - tw * DS;
      const bool ok = pv && (unsigned)ho < (unsigned)g.OH && (unsigned)wo < (unsigned)g.OW;
      const float* bp = dzb + (ok ? ho * g.OW + wo : 0);
      bm = 0;
#pragma unroll
      for (int r = 0; r < TS::B_PER_T; ++r) {
        const int o = o0 + krow0 + KSTEP * r;
        const bool okr = ok && o < g.OC;
        rb[r] = bp[(int64_t)(okr ? o : 0) * g.OHW];
        bm |= (uint32_t)okr << r;
      }
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
  gemm_mainloop<TS>(lds, kbeg, kend, [&](int64_t k0) { load((int)k0); }, store, acc, wm, wn, wk,
                    lane);
  reduce_wk<TS>(acc, lds, wm, wn, wk, lane);
  if (wk == 0) {
#pragma unroll
    for (int aj = 0; aj < TS::RN; ++aj) {
      const int p = n0 + acc_n0<TS>(wn, aj) + acc_col(lane);
      if (p >= npix) continue;
      const int b = p / (HH * WW);
      const int r2 = p - b * HH * WW;
      const int hh = r2 / WW, ww = r2 - hh * WW;
      const int h = ph + S * hh, w = pw + S * ww;
      const int64_t pix_off = (int64_t)b * g.xs + h * g.W + w;
      float* dst = ksplits == 1 ? dx + pix_off : ws + (int64_t)split * g.N * g.xs + pix_off;
#pragma unroll
      for (int ai = 0; ai < TS::RM; ++ai) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = m0 + acc_m0<TS>(wm, ai) + acc_row(r, lane);
          if (i < g.C) {
            float* d = dst + (int64_t)i * g.HW;
            const float v = acc.v[ai][aj][r];
            *d = (ksplits == 1 && accumulate) ? *d + v : v;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Input gradient of a 3x3, pad-1 convolution at stride 1 or 2 ("tile-direct"); at
// stride 1 also dilation DIL = 2 with pad 2 (the halo and the tap offsets scale by DIL,
// a compile-time constant so that the offsets stay immediates).
// The GEMM above fetches dz once per tap; here a work-group stages one dz tile
// (with its halo) and the matching weights in LDS per chunk of 16 output
// channels and runs all nine taps from LDS, so every dz element crosses the
// memory system once per work-group instead of nine times.
//
// A fragment is 32 input pixels that take the same taps; lane l of the MFMA B
// operand reads pixel l of a fragment at LDS address base(pixel) + tap offset,
// the tap offset being a compile-time constant (stride 2) or a uniform value.
//   S = 1: a work-group owns 128*F consecutive pixels (row-major) of one image
//          of width <= 62; wave w owns fragments w*F .. w*F+F-1.
//   S = 2: a work-group owns an 8*FR x 64 region; each wave owns, for each of
//          the four phases (h mod 2, w mod 2), FR phase rows of 32 pixels, so
//          the waves do equal work (the phases take 1, 2, 2 and 4 taps).
// Each fragment accumulates RM blocks of 32 input channels.  No split over K:
// a work-group sums all output channels in a fixed order.
// ---------------------------------------------------------------------------
template <int S, int F, int RM>
struct Dx3Cfg {
  // output channels per LDS chunk
  static constexpr int OCB = (S == 1) ? 8 : 16, BMC = 32 * RM, BMCP = BMC + 1;
  static constexpr int NFRAG = (S == 1) ? F : 4 * F;       // fragments per wave
  // stride 2: region 8F rows x 64 cols -> dz tile (4F + 1) rows x 33 cols
  static constexpr int ZC2 = 33, ZR2 = 4 * F + 1;
  // LDS floats per channel plane (odd): stride 1 holds (rows spanned + 2) x (W + 2),
  // checked on the host (dx3_s1_fits); stride 2 holds the fixed tile
  static constexpr int ZPLANE = (S == 1) ? 513 : ZR2 * ZC2;
  static constexpr int ZFLOATS = OCB * ZPLANE;
  static constexpr int WFLOATS = 9 * OCB * BMC;
  static constexpr int ZPT = (ZFLOATS + kThreads - 1) / kThreads;   // staging registers
  static constexpr int WPT = (OCB * BMC * 9 + kThreads - 1) / kThreads;
};

// Stride-1 tile of 128*F pixels of a W-wide image spans at most floor((128F-1)/W) + 2
// rows; with the halo of a 3x3 window at dilation D the dz tile is (that + 2D) x (W + 2D).
static bool dx3_s1_fits(int W, int F, int zplane, int D = 1) {
  if (W < 8 || W + 2 * D > 64) return false;
  const int rows = (128 * F - 1) / W + 2;
  return (rows + 2 * D) * (W + 2 * D) <= zplane;
}

// Source of the zero padding staged by the LDS-DMA loads (never written).
__device__ float g_dx3_zero[4];


// DMA = true stages each chunk with direct global-to-LDS loads into one of two
// LDS buffers (the next chunk lands while the matrix cores work on this one;
// needs 16-byte aligned weights); DMA = false stages through registers.
// Z4 (DMA, dz width a multiple of 4, 16-byte aligned dz): the dz tile is copied
// in 16-byte pieces (a quarter of the copy instructions); its rows span columns
// -4 .. W+3 at stride 1 and 36 columns at stride 2.
template <int S, int F, int RM, bool DMA, bool Z4, int DIL = 1>
__global__ __launch_bounds__(kThreads, 2) void conv_dx3_direct(ConvGeom g, const float* __restrict__ wt,
                                                            const float* __restrict__ dz,
                                                            float* __restrict__ dx,
                                                            float* __restrict__ ws,
                                                            int accumulate, int tiles_per_img,
                                                            int tiles_w, int ksplits) {
  using C = Dx3Cfg<S, F, RM>;
  static_assert(!Z4 || DMA, "16-byte tile copies are direct copies");
  // group blockIdx.y of a grouped convolution (g holds the group's channel counts and
  // the whole tensors' image strides; 0 on a plain one)
  wt += blockIdx.y * g.gw;
  dz += blockIdx.y * g.gz;
  dx += blockIdx.y * g.gx;
  if (ws) ws += blockIdx.y * g.gx;
  // stride 2 with 16-byte copies: tile columns zc0 .. zc0+35 (nine pieces)
  constexpr int ZC2 = (S == 2 && Z4) ? 36 : C::ZC2;
  constexpr int ZFL = S == 2 ? C::OCB * C::ZR2 * ZC2 : C::ZFLOATS;   // tile floats, at most
  // whole copy blocks: 64 floats (4-byte copies) or 256 floats (16-byte copies)
  constexpr int ZBUF = Z4 ? (ZFL + 255) / 256 * 256 : (ZFL + 63) / 64 * 64;
  // two buffers as separate arrays, so that reads of one provably do not alias
  // the copies in flight into the other
  __shared__ float Z[ZBUF], Z1[DMA ? ZBUF : 1];
  __shared__ float Wl[C::WFLOATS], Wl1[DMA ? C::WFLOATS : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, khalf = lane >> 5;
  const int ctiles = (g.C + C::BMC - 1) / C::BMC;
  // XCD-aware order: the channel tiles and K splits of one pixel tile, which copy
  // the same dz tile, and then the neighbouring pixel tiles run on one XCD (one L2)
  const int bid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int ctile = bid % ctiles;
  const int split = (bid / ctiles) % ksplits;
  const int t = bid / (ctiles * ksplits);
  const int b = t / tiles_per_img, tt = t - b * tiles_per_img;
  const int i0 = ctile * C::BMC;

  // ---- geometry of the dz tile and of this lane's pixels
  int zr0, zc0, ZR, ZC;        // tile origin in dz, tile size
  int pbase[C::NFRAG];         // LDS offset of the lane's pixel (tap (1,1) at stride 1)
  int ph_[C::NFRAG], pw_[C::NFRAG], prow[C::NFRAG], pcol[C::NFRAG];
  bool pval[C::NFRAG];
  if constexpr (S == 1) {
    // dilation D (pad D): tap (kh, kw) reads dz[h + D(1-kh)][w + D(1-kw)]
    constexpr int D = DIL;
    const int p0 = tt * 128 * F;                       // first pixel of the tile
    const int hmin = p0 / g.W;
    zr0 = hmin - D;
    zc0 = Z4 ? -4 : -D;
    ZC = Z4 ? g.W + 8 : g.W + 2 * D;
    const int plast = min(p0 + 128 * F, g.H * g.W) - 1;
    ZR = plast / g.W - hmin + 1 + 2 * D;
#pragma unroll
    for (int f = 0; f < C::NFRAG; ++f) {
      const int p = p0 + (wave * F + f) * 32 + col;
      const int h = p / g.W, w = p - h * g.W;
      pval[f] = p < g.H * g.W;
      prow[f] = h;
      pcol[f] = w;
      // dz[h+D-D kh][w+D-D kw] sits at Z row (h-hmin) + D(2-kh), col w + D(2-kw)
      // (+ 4-D with Z4, whose rows start at column -4)
      pbase[f] = pval[f] ? (h - hmin) * ZC + w + (Z4 ? 4 - D : 0) : 0;
      ph_[f] = pw_[f] = 0;
    }
  } else {
    const int th = tt / tiles_w, tw = tt - th * tiles_w;
    const int h0 = th * 8 * F, w0 = tw * 64;
    zr0 = h0 / 2;
    zc0 = w0 / 2;   // a multiple of 32
    ZR = C::ZR2;
    ZC = ZC2;
#pragma unroll
    for (int f = 0; f < C::NFRAG; ++f) {
      const int phase = f % 4, fr = f / 4;             // fragment = (phase, phase row)
      const int ph = phase >> 1, pw = phase & 1;
      const int rr = wave * F + fr;                    // phase row within the region
      const int h = h0 + 2 * rr + ph, w = w0 + pw + 2 * col;
      pval[f] = h < g.H && w < g.W;
      prow[f] = h;
      pcol[f] = w;
      ph_[f] = ph;
      pw_[f] = pw;
      // dz[(h+1-kh)/2][(w+1-kw)/2] sits at Z row rr + (ph+1-kh)/2, col col + (pw+1-kw)/2
      pbase[f] = rr * ZC2 + col;
    }
  }

  // ---- staging of one chunk (OCB output channels): the dz tile and the weights
  // [o][i][tap].  The host guarantees C % BMC == 0 and OC % OCB == 0, so only
  // the image border masks.  A staged element's offset inside a chunk does not
  // depend on the chunk: computed once (-1 = zero padding).  Unit e of the tile
  // (one float, or a 16-byte piece with Z4) is staged by thread e % 256
  // (wave-contiguous blocks of 64 units).  Planes are ZR*ZC floats apart (dense).
  const int ZP = ZR * ZC;
  const float* dzb = dz + (int64_t)b * g.zs;
  const int zcount = C::OCB * ZP;
  constexpr int ZU = Z4 ? 4 : 1;   // floats per staged unit
  constexpr int ZQ = Z4 ? (ZFL / 4 + kThreads - 1) / kThreads : C::ZPT;
  int zofs[ZQ];
#pragma unroll
  for (int r = 0; r < ZQ; ++r) {
    const int e = (tid + kThreads * r) * ZU;
    const int o = e / ZP, rem = e - o * ZP;
    const int zr = rem / ZC, zc = rem - zr * ZC;
    const int ho = zr0 + zr, wo = zc0 + zc;
    const bool ok = e < zcount && zr < ZR && (unsigned)ho < (unsigned)g.OH &&
                    (unsigned)wo < (unsigned)g.OW;
    zofs[r] = ok ? o * g.OHW + ho * g.OW + wo : -1;
  }
  float rz[DMA ? 1 : C::ZPT], rw[DMA ? 1 : C::WPT];
  // DMA: each wave copies its 64-float blocks of the tile (padding read from the
  // zero page) and its 256-float blocks of the weights straight into LDS buffer `buf`.
  auto issue = [&](int o0, float* zl, float* wl) {
    const float* zb = dzb + (int64_t)o0 * g.OHW;
#pragma unroll
    for (int r = 0; r < ZQ; ++r) {
      const int q = wave + 4 * r;
      int zo = zofs[r];
      asm volatile("" : "+v"(zo));   // keeps the 64-bit addresses from being hoisted
      if (64 * ZU * q < zcount) {
        const float* src = zo >= 0 ? zb + zo : g_dx3_zero;
        if constexpr (Z4)
          __builtin_amdgcn_global_load_lds(src, lds_ptr(zl + 256 * q), 16, 0, 0);
        else
          __builtin_amdgcn_global_load_lds(src, lds_ptr(zl + 64 * q), 4, 0, 0);
      }
    }
    const float* wb = wt + ((int64_t)o0 * g.C + i0) * 9;
    constexpr int WQ = C::WFLOATS / 256;
#pragma unroll
    for (int r = 0; r < (WQ + 3) / 4; ++r) {
      const int q = wave + 4 * r;
      if (q < WQ) {
        const int e = 4 * (64 * q + lane);
        const int o = e / (C::BMC * 9), rem = e - o * (C::BMC * 9);
        __builtin_amdgcn_global_load_lds(wb + o * g.C * 9 + rem, lds_ptr(wl + 256 * q), 16, 0, 0);
      }
    }
  };
  // registers: the loaded values are consumed only by the LDS store of the next
  // chunk (the zero padding is applied there), so the loads stay in flight during
  // the matrix-core work.
  auto load = [&](int o0) {
    const float* zb = dzb + (int64_t)o0 * g.OHW;
#pragma unroll
    for (int r = 0; r < ZQ; ++r) rz[DMA ? 0 : r] = zb[(unsigned)max(zofs[r], 0)];
    const float* wb = wt + ((int64_t)o0 * g.C + i0) * 9;
#pragma unroll
    for (int r = 0; r < C::WPT; ++r) {
      const int e = tid + kThreads * r;                // (o, i, tap), tap fastest
      const int o = e / (C::BMC * 9), rem = e - o * (C::BMC * 9);
      const bool ok = e < C::OCB * C::BMC * 9;
      rw[DMA ? 0 : r] = wb[(unsigned)(ok ? o * g.C * 9 + rem : 0)];
    }
  };
  // LDS keeps the staging order: Z planes of ZR*ZC floats, weights as [o][i][tap]
  // (a lane reads weights 9 floats apart: no bank conflicts).
  auto store = [&]() {
#pragma unroll
    for (int r = 0; r < ZQ; ++r) {
      const int e = tid + kThreads * r;
      if (e < zcount) Z[e] = zofs[r] >= 0 ? rz[DMA ? 0 : r] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < C::WPT; ++r) {
      const int e = tid + kThreads * r;
      if (e < C::OCB * C::BMC * 9) Wl[e] = rw[DMA ? 0 : r];
    }
  };
  f32x16 acc[C::NFRAG][RM];
#pragma unroll
  for (int f = 0; f < C::NFRAG; ++f)
#pragma unroll
    for (int m = 0; m < RM; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][m][r] = 0.f;

  // All taps of one chunk from LDS buffer (zl, wl).  The operands of tap t + 1
  // are read into the other register set while the matrix cores work on tap t.
  // Stride 2: a tap feeds only the fragments of the phases it reaches.
  auto tap_hits = [&](int f, int kh, int kw) {
    return S == 1 || (((ph_[f] + 1 - kh) & 1) == 0 && ((pw_[f] + 1 - kw) & 1) == 0);
  };
  auto compute = [&](const float* zl, const float* wl) {
    constexpr int KK = C::OCB / 2;
    float av[2][KK][RM], bv[2][KK][C::NFRAG];
    auto fetch = [&](int tap, int sl) {
      const int kh = tap / 3, kw = tap - 3 * kh;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int o = 2 * kk + khalf;
#pragma unroll
        for (int m = 0; m < RM; ++m) av[sl][kk][m] = wl[(o * C::BMC + m * 32 + col) * 9 + tap];
#pragma unroll
        for (int f = 0; f < C::NFRAG; ++f) {
          if (!tap_hits(f, kh, kw)) continue;
          int off;
          if constexpr (S == 1)
            off = DIL * ((2 - kh) * ZC + (2 - kw));
          else
            off = ((ph_[f] + 1 - kh) >> 1) * ZC2 + ((pw_[f] + 1 - kw) >> 1);
          bv[sl][kk][f] = zl[o * ZP + pbase[f] + off];
        }
      }
    };
    // per tap: fragments hit, operand reads of the next tap, matrix instructions
    constexpr int HITS = S == 1 ? C::NFRAG : C::NFRAG / 4;
    constexpr int NRD = KK * (RM + HITS), NMF = KK * HITS * RM;
    fetch(0, 0);
#pragma unroll
    for (int tap = 0; tap < 9; ++tap) {
      const int kh = tap / 3, kw = tap - 3 * kh, sl = tap & 1;
      __builtin_amdgcn_sched_barrier(0);
      if (tap < 8) fetch(tap + 1, sl ^ 1);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int f = 0; f < C::NFRAG; ++f) {
          if (!tap_hits(f, kh, kw)) continue;
#pragma unroll
          for (int m = 0; m < RM; ++m)
            acc[f][m] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[sl][kk][m], bv[sl][kk][f],
                                                             acc[f][m], 0, 0, 0);
        }
      // issue all reads of the next tap first, then this tap's matrix work
      if (tap < 8) __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // this split's output-channel chunks [c0, c1)
  const int nch = (g.OC + C::OCB - 1) / C::OCB;
  const int cps = (nch + ksplits - 1) / ksplits;
  const int c0 = min(nch, split * cps), c1 = min(nch, c0 + cps);
  if constexpr (DMA) {
    // chunks alternate between the buffers (Z, Wl) and (Z1, Wl1).  Before each
    // chunk: this wave's copies of it have landed; after the barrier everyone's
    // have, and every wave is done with the previous chunk, whose buffer is
    // refilled next.
    if (c0 < c1) issue(c0 * C::OCB, Z, Wl);
    for (int c = c0; c < c1; c += 2) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (c + 1 < c1) issue((c + 1) * C::OCB, Z1, Wl1);
      compute(Z, Wl);
      if (c + 1 >= c1) break;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (c + 2 < c1) issue((c + 2) * C::OCB, Z, Wl);
      compute(Z1, Wl1);
    }
  } else {
    if (c0 < c1) {
      load(c0 * C::OCB);
      store();
    }
    __syncthreads();
    for (int c = c0; c < c1; ++c) {
      if (c + 1 < c1) load((c + 1) * C::OCB);   // in flight during the matrix-core work
      compute(Z, Wl);
      __syncthreads();
      if (c + 1 < c1) {
        store();
        __syncthreads();
      }
    }
  }


  // ---- epilogue: lane holds pixel `col` of each fragment, channels acc_row(r)
  // with several splits each writes its partial at the pixel's dx position in ws[split]
  float* out = ksplits == 1 ? dx : ws + (int64_t)split * g.N * g.xs;
  const bool add = ksplits == 1 && accumulate;
  if constexpr (S == 2 && DMA) {
    // Stride 2: a fragment's pixels are two columns apart, so the region is first
    // put back in row order in LDS, 8 channels at a time ([8][8F][64] floats in
    // the weight buffer), and written as whole 16-byte row pieces.
    constexpr int RR = 8 * F, TP = 64, CH = 8;
    static_assert(CH * RR * TP <= C::WFLOATS, "epilogue tile exceeds the weight buffer");
    constexpr int NV = CH * RR * TP / 4 / kThreads;   // float4 per thread per pass
    const int th = tt / tiles_w, tw = tt - th * tiles_w;
    const int h0 = th * 8 * F, w0 = tw * 64;
    const bool vec = (g.W % 4) == 0 && ((uintptr_t)out % 16) == 0;
#pragma unroll
    for (int m = 0; m < RM; ++m)
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        __syncthreads();   // the buffer is free (matrix work or previous pass done)
#pragma unroll
        for (int f = 0; f < C::NFRAG; ++f) {
          const int rr = 2 * (wave * F + f / 4) + ph_[f], cc = 2 * col + pw_[f];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            Wl[((4 * khalf + j) * RR + rr) * TP + cc] = acc[f][m][4 * pass + j];
        }
        __syncthreads();
        const int ib = i0 + m * 32 + 8 * pass;   // channels ib .. ib+7 (acc_row of pass)
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          const int u = tid + kThreads * k;
          const int il = u / (RR * TP / 4), rem = u - il * (RR * TP / 4);
          const int rr = rem / (TP / 4), c4 = rem - rr * (TP / 4);
          const int h = h0 + rr, w = w0 + 4 * c4;
          if (h >= g.H || w >= g.W) continue;
          const float4 v = *reinterpret_cast<const float4*>(&Wl[(il * RR + rr) * TP + 4 * c4]);
          float* q = out + (int64_t)b * g.xs + ((int64_t)(ib + il) * g.H + h) * g.W + w;
          if (vec && w + 3 < g.W) {
            float4 o = v;
            if (add) {
              const float4 a = *reinterpret_cast<const float4*>(q);
              o.x += a.x; o.y += a.y; o.z += a.z; o.w += a.w;
            }
            *reinterpret_cast<float4*>(q) = o;
          } else {
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (w + e < g.W) q[e] = add ? q[e] + vv[e] : vv[e];
          }
        }
      }
    return;
  }
#pragma unroll
  for (int f = 0; f < C::NFRAG; ++f) {
    if (!pval[f]) continue;
    float* d = out + (int64_t)b * g.xs + prow[f] * g.W + pcol[f];
#pragma unroll
    for (int m = 0; m < RM; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + m * 32 + acc_row(r, lane);
        if (i < g.C) {
          float* q = d + (int64_t)i * g.HW;
          *q = add ? *q + acc[f][m][r] : acc[f][m][r];
        }
      }
  }
}

// Persistent form of the stride-2 tile-direct dX (16-byte tile copies, no split
// over output channels, NCH chunks of 16 output channels per tile).  Each
// work-group walks the tiles blockIdx.x, blockIdx.x + gridDim.x, ... as one
// sequence of chunk steps: the first chunk of the next tile is copied while the
// last chunk of this one is computed.  Output positions off the image store to
// a sink, so every thread issues the same number of stores per tile.  The wait
// for the next tile's first chunk counts past those stores, but the barrier after
// it (its memory fence) waits for every store in flight anyway, and that full
// wait is what makes the copies safe to read: a count that stops short of
// younger stores does not prove older copies into LDS landed.
__device__ float g_dx3_sink[4 * kThreads];

//
// BA != kFzOff (the activation of the block below, kFzAny: ba.act at run time;
// one 32-channel tile column, 16-byte rows): dx is the delta of a block below
// with batch statistics, and the epilogue also adds up that block's act/BN sums
// sum g and sum g*x_norm, g = dx * act'(y), over the elements it stores: the y
// and x_norm pieces at a pass's store positions are loaded before the pass's
// regroup, each thread keeps the sums of its 16 (pass, piece) channel slots over
// all its tiles, and at the end the work-group adds them up (a fixed shuffle tree
// per wave, then the two waves of a channel in order) into ba.part[c][blockIdx.x].
// ba.apply: the stores hold g itself (the block below's activation step done).
template <int NCH, int BA = kFzOff>
__global__ __launch_bounds__(kThreads, 2) void conv_dx3_s2p(ConvGeom g,
                                                           const float* __restrict__ wt,
                                                           const float* __restrict__ dz,
                                                           float* __restrict__ dx, int accumulate,
                                                           int ntiles, int tiles_per_img,
                                                           int tiles_w, BnBelow ba) {
  using C = Dx3Cfg<2, 1, 1>;
  constexpr bool sums = BA != kFzOff;
  float ss[sums ? 16 : 1][2];
#pragma unroll
  for (int j = 0; j < (sums ? 16 : 1); ++j) ss[j][0] = ss[j][1] = 0.f;
  static_assert(NCH % 2 == 0, "chunks alternate between the two buffers within a tile");
  constexpr int OCB = C::OCB, BMC = C::BMC, NFRAG = C::NFRAG;   // 16, 32, 4
  constexpr int ZC2 = 36, ZR2 = C::ZR2, ZP = ZR2 * ZC2, ZFL = OCB * ZP;
  constexpr int ZBUF = (ZFL + 255) / 256 * 256;
  constexpr int ZQ = (ZFL / 4 + kThreads - 1) / kThreads;   // 16-byte pieces per thread
  constexpr int WQ = C::WFLOATS / 256;                      // 16-byte weight copies per WG
  constexpr int RR = 8, TP = 64, CH = 8, NV = CH * RR * TP / 4 / kThreads;
  constexpr int NST = 4 * NV;                               // stores per thread per tile
  __shared__ float Z[ZBUF], Z1[ZBUF];
  __shared__ float Wl[C::WFLOATS], Wl1[C::WFLOATS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, khalf = lane >> 5;
  const int ctiles = g.C / BMC;

  // fragment f = output phase (ph, pw), phase row = wave: the same in every tile
  int pbase[NFRAG], ph_[NFRAG], pw_[NFRAG];
#pragma unroll
  for (int f = 0; f < NFRAG; ++f) {
    ph_[f] = (f >> 1) & 1;
    pw_[f] = f & 1;
    pbase[f] = wave * ZC2 + col;
  }
  struct Tile {
    int b, i0, h0, w0;
  };
  auto tile_of = [&](int t) {
    Tile r;
    const int ct = t % ctiles, pt = t / ctiles;
    r.b = pt / tiles_per_img;
    const int tp = pt - r.b * tiles_per_img, th = tp / tiles_w;
    r.h0 = th * 8;
    r.w0 = (tp - th * tiles_w) * 64;
    r.i0 = ct * BMC;
    return r;
  };
  // source offsets of this thread's tile pieces for tile `nt` (-1: zero padding)
  int zofs[ZQ];
  auto set_zofs = [&](const Tile& nt) {
    const int zr0 = nt.h0 / 2, zc0 = nt.w0 / 2;
#pragma unroll
    for (int r = 0; r < ZQ; ++r) {
      const int e = (tid + kThreads * r) * 4;
      const int o = e / ZP, rem = e - o * ZP;
      const int zr = rem / ZC2, zc = rem - zr * ZC2;
      const int ho = zr0 + zr, wo = zc0 + zc;
      const bool ok = e < ZFL && (unsigned)ho < (unsigned)g.OH && (unsigned)wo < (unsigned)g.OW;
      zofs[r] = ok ? o * g.OHW + ho * g.OW + wo : -1;
    }
  };
  auto issue = [&](const Tile& nt, int chunk, float* zl, float* wl) {
    const float* zb = dz + ((int64_t)nt.b * g.OC + chunk * OCB) * g.OHW;
#pragma unroll
    for (int r = 0; r < ZQ; ++r) {
      const int q = wave + 4 * r;
      int zo = zofs[r];
      asm volatile("" : "+v"(zo));   // keeps the 64-bit addresses from being hoisted
      if (256 * q < ZFL)
        __builtin_amdgcn_global_load_lds(zo >= 0 ? zb + zo : g_dx3_zero, lds_ptr(zl + 256 * q),
                                         16, 0, 0);
    }
    const float* wb = wt + ((int64_t)chunk * OCB * g.C + nt.i0) * 9;
#pragma unroll
    for (int r = 0; r < (WQ + 3) / 4; ++r) {
      const int q = wave + 4 * r;
      if (q < WQ) {
        const int e = 4 * (64 * q + lane);
        const int o = e / (BMC * 9), rem = e - o * (BMC * 9);
        __builtin_amdgcn_global_load_lds(wb + o * g.C * 9 + rem, lds_ptr(wl + 256 * q), 16, 0, 0);
      }
    }
  };

  f32x16 acc[NFRAG];
  auto zero_acc = [&]() {
#pragma unroll
    for (int f = 0; f < NFRAG; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][r] = 0.f;
  };
  auto tap_hits = [&](int f, int kh, int kw) {
    return ((ph_[f] + 1 - kh) & 1) == 0 && ((pw_[f] + 1 - kw) & 1) == 0;
  };
  // all taps of one chunk; tap t+1's operands are read while tap t's matrix work runs
  auto compute = [&](const float* zl, const float* wl) {
    constexpr int KK = OCB / 2;
    float av[2][KK], bv[2][KK][NFRAG];
    auto fetch = [&](int tap, int sl) {
      const int kh = tap / 3, kw = tap - 3 * kh;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int o = 2 * kk + khalf;
        av[sl][kk] = wl[(o * BMC + col) * 9 + tap];
#pragma unroll
        for (int f = 0; f < NFRAG; ++f) {
          if (!tap_hits(f, kh, kw)) continue;
          const int off = ((ph_[f] + 1 - kh) >> 1) * ZC2 + ((pw_[f] + 1 - kw) >> 1);
          bv[sl][kk][f] = zl[o * ZP + pbase[f] + off];
        }
      }
    };
    constexpr int NRD = KK * 2, NMF = KK;   // one fragment per tap
    fetch(0, 0);
#pragma unroll
    for (int tap = 0; tap < 9; ++tap) {
      const int kh = tap / 3, kw = tap - 3 * kh, sl = tap & 1;
      __builtin_amdgcn_sched_barrier(0);
      if (tap < 8) fetch(tap + 1, sl ^ 1);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int f = 0; f < NFRAG; ++f) {
          if (!tap_hits(f, kh, kw)) continue;
          acc[f] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[sl][kk], bv[sl][kk][f], acc[f], 0, 0, 0);
        }
      if (tap < 8) __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // The tile's 8 x 64 output region, 8 channels at a time, regrouped in row
  // order in the free weight buffer `buf` and stored in 16-byte pieces; every
  // thread issues NST stores (positions off the image go to the sink).
  const bool vec = (g.W % 4) == 0 && ((uintptr_t)dx % 16) == 0;
  auto epilogue = [&](const Tile& ct, float* buf) {
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      // the block below's y and x_norm at this pass's store positions, in flight
      // during the regroup
      float4 yv[sums ? NV : 1], xv[sums ? NV : 1];
      if constexpr (sums) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          const int u = tid + kThreads * k;
          const int il = u / (RR * TP / 4), rem = u - il * (RR * TP / 4);
          const int rr = rem / (TP / 4), c4 = rem - rr * (TP / 4);
          const int h = ct.h0 + rr, w = ct.w0 + 4 * c4;
          const int64_t o = h < g.H && w + 3 < g.W
                                ? (((int64_t)ct.b * g.C + ct.i0 + 8 * pass + il) * g.H + h) * g.W + w
                                : 0;
          yv[k] = *reinterpret_cast<const float4*>(ba.y + o);
          xv[k] = *reinterpret_cast<const float4*>(ba.xn + o);
        }
      }
      __syncthreads();   // the buffer is free (matrix work or previous pass done)
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        const int rr = 2 * wave + ph_[f], cc = 2 * col + pw_[f];
#pragma unroll
        for (int j = 0; j < 4; ++j) buf[((4 * khalf + j) * RR + rr) * TP + cc] = acc[f][4 * pass + j];
      }
      __syncthreads();
      const int ib = ct.i0 + 8 * pass;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int u = tid + kThreads * k;
        const int il = u / (RR * TP / 4), rem = u - il * (RR * TP / 4);
        const int rr = rem / (TP / 4), c4 = rem - rr * (TP / 4);
        const int h = ct.h0 + rr, w = ct.w0 + 4 * c4;
        float4 v = *reinterpret_cast<const float4*>(&buf[(il * RR + rr) * TP + 4 * c4]);
        float* q = dx + (((int64_t)ct.b * g.C + ib + il) * g.H + h) * g.W + w;
        const bool whole = h < g.H && w + 3 < g.W && vec;
        if (!whole && h < g.H && w < g.W) {
          // ragged right edge or unaligned rows: element stores, then the sink
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (w + e < g.W) q[e] = accumulate ? q[e] + vv[e] : vv[e];
        }
        float4* d = whole ? reinterpret_cast<float4*>(q) : reinterpret_cast<float4*>(g_dx3_sink) + tid;
        if (accumulate && whole) {
          const float4 a = *d;
          v.x += a.x; v.y += a.y; v.z += a.z; v.w += a.w;
        }
        if constexpr (sums) {
          const int act = BA == kFzAny ? ba.act : BA;
          const float g0 = v.x * act_grad(act, ba.slope, yv[k].x);
          const float g1 = v.y * act_grad(act, ba.slope, yv[k].y);
          const float g2 = v.z * act_grad(act, ba.slope, yv[k].z);
          const float g3 = v.w * act_grad(act, ba.slope, yv[k].w);
          if (whole) {
            ss[4 * pass + k][0] += (g0 + g1) + (g2 + g3);
            ss[4 * pass + k][1] += (g0 * xv[k].x + g1 * xv[k].y) + (g2 * xv[k].z + g3 * xv[k].w);
          }
          if (ba.apply) v = make_float4(g0, g1, g2, g3);   // the delta below, act step done
        }
        *d = v;
      }
    }
  };

  const int mytiles = (ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  if (mytiles <= 0) return;
  Tile cur = tile_of(blockIdx.x);
  set_zofs(cur);
  issue(cur, 0, Z, Wl);
  // the same count of younger stores as after a tile, so the first wait below
  // looks like every later one
  {
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < NST; ++k) reinterpret_cast<float4*>(g_dx3_sink)[tid] = zero4;
  }
  for (int k = 0; k < mytiles; ++k) {
    const int tn = blockIdx.x + (k + 1 < mytiles ? k + 1 : k) * gridDim.x;   // next (or this) tile
    const Tile nxt = tile_of(tn);
    zero_acc();
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float* zr = (c & 1) ? Z1 : Z;
      float* wr = (c & 1) ? Wl1 : Wl;
      float* zn = (c & 1) ? Z : Z1;
      float* wn = (c & 1) ? Wl : Wl1;
      // this wave's copies of chunk c have landed (at c == 0 once the barrier's fence
      // has waited for the stores too); after the barrier everyone's have, and the
      // other buffer is free
      static_assert(NST == 16, "the wait below counts 16 stores");
      if (c == 0)
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (c + 1 < NCH) {
        issue(cur, c + 1, zn, wn);
      } else {
        set_zofs(nxt);
        issue(nxt, 0, zn, wn);
      }
      compute(zr, wr);
    }
    // chunk NCH-1 used buffer 1 (NCH even): its weight buffer is free for the regroup
    epilogue(cur, Wl1);
    cur = nxt;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // nothing in flight at exit
  if constexpr (sums) {
    // thread tid holds channel 8 pass + 2 k + (tid >> 7) in slot 4 pass + k: waves 0-1
    // the even channels, waves 2-3 the odd ones
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float v = ss[j][e];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        ss[j][e] = v;
      }
    __syncthreads();   // every wave is past its last use of the LDS buffers
    float* red = Z;    // [wave][slot][2]
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        red[(wave * 16 + j) * 2] = ss[j][0];
        red[(wave * 16 + j) * 2 + 1] = ss[j][1];
      }
    }
    __syncthreads();
    if (tid < 64) {
      const int c = tid >> 1, e = tid & 1, par = c & 1;
      const int j = 4 * (c >> 3) + ((c & 7) >> 1);
      const float v = red[((2 * par) * 16 + j) * 2 + e] + red[((2 * par + 1) * 16 + j) * 2 + e];
      reinterpret_cast<float*>(ba.part + (int64_t)c * gridDim.x + blockIdx.x)[e] = v;
    }
  }
}

// Input gradient from the column buffer (the pages' route: P1 section 3.1's
// gemm(1,0,...) of W^T and delta, then section 3.2's col2im):
// dx[n][i][h][w] (+)= sum over (kh, kw), in that order, of col[n][(i,kh,kw)][ho][wo]
// with ho*S = h + P - kh, wo*S = w + P - kw on the map (dense layers).
// S1: stride 1, where the taps that reach an element form one rectangle
// kh in [h + P - OH + 1, h + P], kw likewise, visited without tests.
template <bool S1>
__global__ __launch_bounds__(kThreads) void col2im_kernel(ConvGeom g, const float* __restrict__ col,
                                                          float* __restrict__ dx, int accumulate) {
  const int64_t total = (int64_t)g.N * g.C * g.HW;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
    const int n = (int)(e / ((int64_t)g.C * g.HW));
    const int rem = (int)(e - (int64_t)n * g.C * g.HW);
    const int i = rem / g.HW, pix = rem - i * g.HW;
    const int h = pix / g.W, w = pix - h * g.W;
    const float* cb = col + ((int64_t)n * g.J + (int64_t)i * g.K * g.K) * g.OHW;
    float s = 0.f;
    if constexpr (S1) {
      const int kh0 = max(0, h + g.P - g.OH + 1), kh1 = min(g.K - 1, h + g.P);
      const int kw0 = max(0, w + g.P - g.OW + 1), kw1 = min(g.K - 1, w + g.P);
      for (int kh = kh0; kh <= kh1; ++kh) {
        const float* r = cb + (int64_t)kh * g.K * g.OHW + (h + g.P - kh) * g.OW + w + g.P;
        for (int kw = kw0; kw <= kw1; ++kw) s += r[kw * (g.OHW - 1)];
      }
    } else {
      for (int kh = 0; kh < g.K; ++kh) {
        const int hn = h + g.P - kh;
        if (hn < 0 || hn % g.S) continue;
        const int ho = hn / g.S;
        if (ho >= g.OH) continue;
        for (int kw = 0; kw < g.K; ++kw) {
          const int wn = w + g.P - kw;
          if (wn < 0 || wn % g.S) continue;
          const int wo = wn / g.S;
          if (wo >= g.OW) continue;
          s += cb[(int64_t)(kh * g.K + kw) * g.OHW + ho * g.OW + wo];
        }
      }
    }
    dx[e] = accumulate ? dx[e] + s : s;
  }
}

// dx[e] (+)= sum over splits s (in order) of ws[s][e].
template <int W>
__global__ __launch_bounds__(kThreads) void dx_splitk_reduce(float* __restrict__ dx,
                                                             const float* __restrict__ ws,
                                                             int splits, int64_t n,
                                                             int accumulate) {
  using V = RedVec<W>;
  const int64_t stride = (int64_t)gridDim.x * kThreads * W;
  for (int64_t e = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * W; e < n; e += stride) {
    const V s = vsum_in_order<W>(ws, 0, splits, n, e);
    V* d = reinterpret_cast<V*>(dx + e);
    *d = accumulate ? *d + s : s;
  }
}

// dx (+)= the ordered sum of the `splits` input-gradient partials in ws.
static int launch_dx_reduce(float* dx, const float* ws, int splits, int64_t n, int accumulate,
                            hipStream_t st) {
  const bool v4 = n % 4 == 0 && (((uintptr_t)dx | (uintptr_t)ws) & 15) == 0 && n >= kRedVecMin;
  const unsigned blocks =
      (unsigned)std::min<int64_t>(ceil_div(v4 ? n / 4 : n, kThreads), 8192);
  if (v4)
    dx_splitk_reduce<4><<<blocks, kThreads, 0, st>>>(dx, ws, splits, n, accumulate);
  else
    dx_splitk_reduce<1><<<blocks, kThreads, 0, st>>>(dx, ws, splits, n, accumulate);
  return check_launch("dx_splitk_reduce", st);
}

// ---------------------------------------------------------------------------
// Input gradient for very few input channels (CI <= 4) at stride 1, e.g. the
// image gradient of a network's first layer.  Such a layer is HBM-bound
// (reads dz with C_out channels, writes only CI), and a matrix-core tile would
// waste all but CI of its 32 rows, so it runs on the vector ALUs:
//   dx[n][i][h][w] = sum_{o,kh,kw} W[o][i][kh][kw] * dz[n][o][h+p-kh][w+p-kw].
// A work-group owns a 16 x 64 pixel tile of one image; dz for 8 output channels
// at a time is staged in LDS with its (K-1) halo, and each thread accumulates 4
// neighbouring pixels of one row for all CI channels.  Weights are read with
// block-uniform addresses.
// ---------------------------------------------------------------------------
constexpr int kScTH = 16, kScTW = 64, kScOCB = 8;

template <int CI, int K>
__global__ __launch_bounds__(kThreads) void conv_dx_smallc_kernel(ConvGeom g,
                                                                  const float* __restrict__ wt,
                                                                  const float* __restrict__ dz,
                                                                  float* __restrict__ dx,
                                                                  int tiles_w, int tiles_h,
                                                                  int accumulate) {
  constexpr int LH = kScTH + K - 1, LW = kScTW + K - 1, LWP = LW + 1;
  __shared__ float tile[kScOCB][LH][LWP];
  const int tid = threadIdx.x;
  const int tw_i = blockIdx.x % tiles_w;
  const int th_i = (blockIdx.x / tiles_w) % tiles_h;
  const int b = blockIdx.x / (tiles_w * tiles_h);
  const int h0 = th_i * kScTH, w0 = tw_i * kScTW;
  const int ho0 = h0 + g.P - (K - 1), wo0 = w0 + g.P - (K - 1);
  const int r = tid / (kScTW / 4), c0 = (tid % (kScTW / 4)) * 4;

  float acc[CI][4];
#pragma unroll
  for (int i = 0; i < CI; ++i)
#pragma unroll
    for (int px = 0; px < 4; ++px) acc[i][px] = 0.f;

  const float* dzb = dz + (int64_t)b * g.OC * g.OHW;
  // Staging: each wave copies whole tile rows, lane = column (and column + 64 for
  // the halo), so the per-element index math is one add.
  const int lane = tid & 63, wave = tid >> 6;
  const int wo_a = wo0 + lane;
  const bool ca = (unsigned)wo_a < (unsigned)g.OW;
  constexpr int ROWS = kScOCB * LH;                  // tile rows per chunk
  constexpr int RB = 6;                              // rows in flight per wave
  for (int ob = 0; ob < g.OC; ob += kScOCB) {
    __syncthreads();
    for (int row0 = wave; row0 < ROWS; row0 += 4 * RB) {
      float v[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int row = row0 + 4 * u;
        const int o = row / LH, rr = row - o * LH;
        const int ho = ho0 + rr;
        const bool ok = row < ROWS && ob + o < g.OC && (unsigned)ho < (unsigned)g.OH && ca;
        const float t = dzb[ok ? (int64_t)(ob + o) * g.OHW + ho * g.OW + wo_a : 0];
        v[u] = ok ? t : 0.f;
      }
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int row = row0 + 4 * u;
        if (row < ROWS) (&tile[0][0][0])[(row / LH) * LH * LWP + (row % LH) * LWP + lane] = v[u];
      }
    }
    // the K-1 halo columns beyond the first 64
    if constexpr (LW > 64) {
      for (int e = tid; e < ROWS * (LW - 64); e += kThreads) {
        const int row = e / (LW - 64), cc = 64 + e % (LW - 64);
        const int o = row / LH, rr = row - o * LH;
        const int ho = ho0 + rr, wo = wo0 + cc;
        const bool ok =
            ob + o < g.OC && (unsigned)ho < (unsigned)g.OH && (unsigned)wo < (unsigned)g.OW;
        const float t = dzb[ok ? (int64_t)(ob + o) * g.OHW + ho * g.OW + wo : 0];
        tile[o][rr][cc] = ok ? t : 0.f;
      }
    }
    __syncthreads();
    const int onum = min(kScOCB, g.OC - ob);
    for (int o = 0; o < onum; ++o) {
      const float* wo_ = wt + (int64_t)(ob + o) * CI * K * K;
#pragma unroll
      for (int kh = 0; kh < K; ++kh) {
        float seg[4 + K - 1];
#pragma unroll
        for (int j = 0; j < 4 + K - 1; ++j) seg[j] = tile[o][r + K - 1 - kh][c0 + j];
#pragma unroll
        for (int kw = 0; kw < K; ++kw) {
#pragma unroll
          for (int i = 0; i < CI; ++i) {
            const float wv = wo_[(i * K + kh) * K + kw];
#pragma unroll
            for (int px = 0; px < 4; ++px) acc[i][px] += wv * seg[px + K - 1 - kw];
          }
        }
      }
    }
  }
  const int h = h0 + r;
  if (h >= g.H) return;
#pragma unroll
  for (int i = 0; i < CI; ++i) {
    float* d = dx + ((int64_t)b * CI + i) * g.HW + (int64_t)h * g.W + w0 + c0;
#pragma unroll
    for (int px = 0; px < 4; ++px) {
      if (w0 + c0 + px < g.W) d[px] = accumulate ? d[px] + acc[i][px] : acc[i][px];
    }
  }
}

// ---------------------------------------------------------------------------
// Weight and input gradients of a 3x3, pad-1, stride-1 convolution with at
// most 3 input and at most 32 output channels (a network's first layer on an
// RGB image) in one streaming pass over dz: both gradients read the same dz
// and the layer is HBM-bound, so fusing them halves its traffic.  Every dz, x
// and dx element crosses HBM once (plus two halo dz rows per run of rows).
//
// A work-group owns (image, strip of SWo <= 120 output columns starting at w0,
// run of rows r0 .. r1-1) and walks the dz rows h = r0-1 .. r1 inside the image.
// LDS column k holds image column w0 - 4 + k (16-byte load groups; the image
// width is a multiple of 4).  Per dz row:
//   dW: matrix cores, M = o (32), N = (i, kh, kw) (9*CI <= 27 of 32 columns),
//       K = the strip's pixels of row h, two per 32x32x2 step; wave w takes the
//       32 pixels w0 - 1 + 32w ..; pixels outside the strip are masked.  Only the
//       rows r0 .. r1-1 count, so each dz row is counted by exactly one run.
//   dX: matrix cores form P[(i,kh,kw)][p] = sum_o W[o][i][kh][kw] dz[o][h][p] for
//       the 128 pixels p = w0 - 1 .. w0 + 126 (M = (i,kh,kw), N = 32 pixels per
//       wave, K = o).  dz[o][h][p] reaches dx[i][h+kh-1][p+kw-1], so after P
//       goes through LDS, strip column c takes, in a fixed order,
//       P[(i,kh,0)][c+1] + P[(i,kh,1)][c] + P[(i,kh,2)][c-1] into dx row
//       h + kh - 1; each dx row stays in registers until its third dz row.
// dz rows and the P block live in two LDS buffers each (row h uses buffer h & 1)
// and x rows in a ring of four (slot = row & 3), so a row needs one barrier: at
// its start each thread stores dz row h+1 and x row h+2 (loaded two rows earlier
// into one of two register sets) into the buffers row h does not read, while the
// other work-group's waves on the CU keep the matrix cores busy, and after its
// matrix work sends the loads for rows h+3 / h+4; the combine of row h reads its
// own P buffer after the barrier.
// ---------------------------------------------------------------------------
// Row pitches, one per LDS array, for the 64 banks that serve a whole wave's 32-bit
// accesses: dz 134 (= 2 mod 4: the dW operand's 32 channel rows at one column fall on
// distinct even banks, its second half-wave's next column on the odd ones), x 132
// (= 4 mod 64: the x operand's rows four banks apart), P 136 (= 8 mod 16: its two
// half-waves write rows four apart, 32 banks apart).  The P step pairs the channels
// o and o + 16 (16 rows of 134 apart: 32 banks) in one 32x32x2 step.  Measured on the
// stem's first layer: bank conflicts in 35% of the LDS-active cycles, against 43% with
// one odd pitch (133) for all three (most of the rest: the staging stores, four
// consecutive floats per lane); the kernel's time is the same either way.
constexpr int kFrThreads = 256, kFrPitch = 134, kFrPitchX = 132, kFrPitchP = 136, kFrMaxW = 120;

//
// FZ != kFzOff: dz is not read back but formed as it is staged, from delta (the
// dz argument), y and x_norm with the per-channel map of the BN backward
// (DzSource): the write and the re-read of dz by a separate pass disappear.  FZ
// is the activation (kFzAny: the run-time src.act), so the per-element
// derivative compiles to straight-line code for the common ones.
template <int CI, bool ACC, int FZ>
__global__ __launch_bounds__(kFrThreads, 2) void conv_first_rows(
    ConvGeom g, const float* __restrict__ x, const float* __restrict__ wt,
    const float* __restrict__ dz, float* __restrict__ dwpart, float* __restrict__ dx,
    int nstrips, int sw, int nruns, int rlen, DzSource src) {
  static_assert(CI >= 1 && CI <= 3, "9*CI columns must fit one 32-wide block");
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int P = kFrPitch, PX = kFrPitchX, PP = kFrPitchP;
  __shared__ float Zs[2][32 * P];
  __shared__ float Xs[4 * CI * PX];
  __shared__ float Ps[2][32 * PP];
  __shared__ float Z0[64];   // zeros: masked operands read here (no branches around reads)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  const int run = bid % nruns, strip = (bid / nruns) % nstrips;
  const int n = bid / (nruns * nstrips);
  const int w0 = strip * sw, r0 = run * rlen, r1 = min(g.H, r0 + rlen);
  // dz rows hA .. hE are walked (row H, past the image, reads as zeros and
  // completes dx row H-1); the count is rounded up to even, and the extra row
  // changes nothing (its dx row is outside the run)
  const int hA = max(r0 - 1, 0), hE = min(r1, g.H);
  const float* zb = dz + (int64_t)n * g.OC * g.HW;
  const float* xb = x + (int64_t)n * CI * g.HW;
  // last 16-byte group of a row that holds a column the strip uses (LDS column sw + 4)
  const int vlast = (sw + 4) >> 2;

  // channels >= OC are never staged and stay zero
  for (int e = tid; e < 2 * 32 * P; e += kFrThreads) (&Zs[0][0])[e] = 0.f;
  if (tid < 64) Z0[tid] = 0.f;
  // x columns 128 .. P-1 are never staged but are read as the dW operand of the
  // masked pixels past the strip (times a zero dz): they must hold zeros, not
  // whatever the LDS held before (0 x NaN is NaN)
  for (int e = tid; e < 4 * CI * (PX - 128); e += kFrThreads)
    Xs[(e / (PX - 128)) * PX + 128 + e % (PX - 128)] = 0.f;

  // ---- staging: thread slot k takes 16-byte group e = tid + 256k of a row
  // (dz: channel e / 32, group e % 32; x: the same with CI channels).  Groups
  // off the image are zero, applied at the LDS store.  Two register sets: the
  // rows loaded during row h are stored to LDS at the start of row h + 2.
  constexpr bool fz = FZ != kFzOff, fz_y = fz && FZ != CBB_ACT_LINEAR;
  struct Stage {
    f4 pz[4], py[fz ? 4 : 1], pn[fz ? 4 : 1], px;
    uint32_t zmask;
    bool xok;
  };
  // FZ: the map of the four channels this thread stages, o = tid / 32 + 8k
  const float* yb = fz_y ? src.y + (int64_t)n * g.OC * g.HW : zb;
  // without x_norm the third coefficient is 0 and delta stands in for it
  const float* nb = fz && src.xn ? src.xn + (int64_t)n * g.OC * g.HW : zb;
  float ca[4], cb[4], cc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int o = (tid >> 5) + 8 * k;
    ca[k] = cb[k] = cc[k] = 0.f;
    if (fz && o < g.OC) {
      ca[k] = src.coef[o];
      cb[k] = src.coef[g.OC + o];
      cc[k] = src.coef[2 * g.OC + o];
    }
  }
  auto load_dz = [&](Stage& q, int h) {
    q.zmask = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = tid + kFrThreads * k, o = e >> 5, v = e & 31;
      const int w = w0 - 4 + 4 * v;
      // only the groups under columns w0-1 .. w0+sw are fetched (the rest stay zero)
      const bool ok = o < g.OC && v <= vlast && (unsigned)h < (unsigned)g.H &&
                      (unsigned)w < (unsigned)g.W;
      const int off = ok ? (o * g.H + h) * g.W + w : 0;
      q.pz[k] = *(const f4*)(zb + off);
      if constexpr (fz_y) q.py[k] = *(const f4*)(yb + off);
      if constexpr (fz) q.pn[k] = *(const f4*)(nb + off);
      q.zmask |= (uint32_t)ok << k;
    }
  };
  auto store_dz = [&](const Stage& q, int buf) {
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = tid + kFrThreads * k, o = e >> 5, v = e & 31;
      if (o < g.OC) {
        f4 val = q.pz[k];
        if constexpr (fz_y) {
          const int act = FZ == kFzAny ? src.act : FZ;
          val.x *= act_grad(act, src.slope, q.py[k].x);
          val.y *= act_grad(act, src.slope, q.py[k].y);
          val.z *= act_grad(act, src.slope, q.py[k].z);
          val.w *= act_grad(act, src.slope, q.py[k].w);
        }
        if constexpr (fz) {
          const f4 xn = q.pn[k];
          val.x = ca[k] * val.x + cb[k] + cc[k] * xn.x;
          val.y = ca[k] * val.y + cb[k] + cc[k] * xn.y;
          val.z = ca[k] * val.z + cb[k] + cc[k] * xn.z;
          val.w = ca[k] * val.w + cb[k] + cc[k] * xn.w;
        }
        val = ((q.zmask >> k) & 1u) ? val : zero;
        float* d = Zs[buf] + o * P + 4 * v;
        d[0] = val.x;
        d[1] = val.y;
        d[2] = val.z;
        d[3] = val.w;
      }
    }
  };
  auto load_x = [&](Stage& q, int h) {
    const int c = tid >> 5, v = tid & 31, w = w0 - 4 + 4 * v;
    q.xok = tid < CI * 32 && v <= vlast && (unsigned)h < (unsigned)g.H &&
            (unsigned)w < (unsigned)g.W;
    q.px = *(const f4*)(xb + (q.xok ? (c * g.H + h) * g.W + w : 0));
  };
  auto store_x = [&](const Stage& q, int h) {
    const int c = tid >> 5, v = tid & 31;
    const f4 zero = {0.f, 0.f, 0.f, 0.f};
    if (tid < CI * 32) {
      const f4 val = q.xok ? q.px : zero;
      float* d = Xs + ((h & 3) * CI + c) * PX + 4 * v;
      d[0] = val.x;
      d[1] = val.y;
      d[2] = val.z;
      d[3] = val.w;
    }
  };

  // ---- matrix-core operands.  Lane: kq = lane / 32, j = lane % 32.
  const int kq = lane >> 5, j = lane & 31;
  const bool jv = j < 9 * CI;
  // P: A = W^T, constant: wa[k] = W[o = k + 16 kq][j]
  float wa[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int o = k + 16 * kq;
    wa[k] = (jv && o < g.OC) ? wt[o * 9 * CI + j] : 0.f;
  }
  // dW: B column j = (i, kh, kw) reads x row h + kh - 1 at column p + kw - 1
  int xi = 0, xkh = 0, xkw = 0;
  if (jv) {
    xi = j / 9;
    const int tap = j - 9 * xi;
    xkh = tap / 3;
    xkw = tap - 3 * xkh;
  }
  f32x16 adw;
#pragma unroll
  for (int r = 0; r < 16; ++r) adw[r] = 0.f;
  // dx rows h-1 and h of strip column w0 + tid (threads tid < sw)
  float dprev[CI], dcur[CI];
#pragma unroll
  for (int i = 0; i < CI; ++i) dprev[i] = dcur[i] = 0.f;
  const int col = w0 + tid;
  const bool cown = tid < sw && col < g.W;
  const int pb = 3 + 32 * wave;   // LDS column of this wave's first pixel w0 - 1 + 32 * wave

  // One dz row.  `q` holds dz row h+1 and x row h+2 on entry; refilled with
  // dz row h+3 and x row h+4.
  auto row = [&](int h, Stage& q) {
    const int zb_ = h & 1;
    // staging is unconditional (rows past the image are zeros): straight-line
    // code keeps the compiler's waits on these loads precise
    store_dz(q, zb_ ^ 1);
    store_x(q, h + 2);
    // dW over this wave's 32 pixels of row h (rows of the run only)
    if (h >= r0 && h < r1) {
      // masked operands (pixels outside the strip, columns j >= 9*CI) read zeros:
      // the address is selected, so every read is unconditional
      const float* xr =
          jv ? Xs + (((h + xkh - 1) & 3) * CI + xi) * PX + pb + xkw - 1 + kq : Z0;
      const float* zr = Zs[zb_] + j * P + pb + kq;
      float av[16], bv[16];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const bool pin = (unsigned)(32 * wave + 2 * s + kq - 1) < (unsigned)sw;
        av[s] = *(pin ? zr + 2 * s : Z0);
        bv[s] = xr[2 * s];
      }
#pragma unroll
      for (int s = 0; s < 16; ++s)
        adw = __builtin_amdgcn_mfma_f32_32x32x2f32(av[s], bv[s], adw, 0, 0, 0);
      // all operand reads in flight before the matrix work starts
      __builtin_amdgcn_sched_group_barrier(0x100, 32, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P for this wave's 32 pixels
    {
      f32x16 ap;
#pragma unroll
      for (int r = 0; r < 16; ++r) ap[r] = 0.f;
      const float* zc = Zs[zb_] + 16 * kq * P + pb + j;
      float zv[16];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 16; ++k) zv[k] = zc[k * P];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        ap = __builtin_amdgcn_mfma_f32_32x32x2f32(wa[k], zv[k], ap, 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) Ps[zb_][acc_row(r, lane) * PP + pb + j] = ap[r];
    }
    // the registers of q are free again (not live across the matrix work)
    load_dz(q, h + 3);
    load_x(q, h + 4);
    // P and the staged rows h+1 / h+2 complete; row h's reads of Zs and Xs are
    // done, so row h+1 may overwrite them (the other buffer, the ring's free slot)
    __syncthreads();
    if (cown) {
      // dx row h-1 is complete after this row; rows h and h+1 take their share
      float qv[CI][3];
      const int k0 = tid + 4;   // LDS column of strip column col
#pragma unroll
      for (int i = 0; i < CI; ++i)
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) {
          const float* pr = Ps[zb_] + (i * 9 + kh * 3) * PP + k0;
          qv[i][kh] = (pr[1] + pr[PP]) + pr[2 * PP - 1];
        }
      const int hp = h - 1;
#pragma unroll
      for (int i = 0; i < CI; ++i) {
        const float vprev = dprev[i] + qv[i][0];
        if (hp >= r0 && hp < r1) {
          float* d = dx + ((int64_t)(n * CI + i) * g.H + hp) * g.W + col;
          *d = ACC ? *d + vprev : vprev;
        }
        dprev[i] = dcur[i] + qv[i][1];
        dcur[i] = qv[i][2];
      }
    }
  };

  // ---- prologue: x rows hA-1 .. hA+1 and dz row hA staged; rows hA+1 and hA+2
  // (x: hA+2 and hA+3) in the two register sets
  Stage s0, s1;
  for (int h = hA - 1; h <= hA + 1; ++h) {
    load_x(s0, h);
    store_x(s0, h);
  }
  load_dz(s0, hA);
  __syncthreads();   // the zero fill is done before the staged rows land
  store_dz(s0, hA & 1);
  load_dz(s0, hA + 1);
  load_x(s0, hA + 2);
  load_dz(s1, hA + 2);
  load_x(s1, hA + 3);
  __syncthreads();

  for (int h = hA; h <= hE; h += 2) {
    row(h, s0);
    row(h + 1, s1);
  }

  // Sum the four waves' dW blocks (fixed order) and write this work-group's partial.
  __syncthreads();
  float* red = Zs[0];  // 4 x 16 x 64 floats
#pragma unroll
  for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = adw[r];
  __syncthreads();
  if (wave == 0) {
    float* dst = dwpart + (int64_t)bid * g.OC * g.J;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = (red[r * 64 + lane] + red[(16 + r) * 64 + lane]) +
                      (red[(32 + r) * 64 + lane] + red[(48 + r) * 64 + lane]);
      const int o = acc_row(r, lane);
      if (o < g.OC && jv) dst[o * g.J + j] = v;
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
  g.G = d.groups > 1 ? d.groups : 1;
  g.D = d.dilation > 1 ? d.dilation : 1;
  const int span = g.D * (d.ksize - 1) + 1;   // input pixels under one window
  g.OH = (d.in_h + 2 * d.pad - span) / d.stride + 1;
  g.OW = (d.in_w + 2 * d.pad - span) / d.stride + 1;
  g.HW = g.H * g.W;
  g.OHW = g.OH * g.OW;
  g.J = g.C / g.G * g.K * g.K;
  g.Q = (int64_t)g.N * g.OHW;
  g.xs = (int64_t)g.C * g.HW;
  g.zs = (int64_t)g.OC * g.OHW;
  g.gx = (int64_t)(g.C / g.G) * g.HW;
  g.gz = (int64_t)(g.OC / g.G) * g.OHW;
  g.gw = (int64_t)(g.OC / g.G) * g.J;
  return g;
}

// A plain convolution: no groups, no dilation, packed image strides.  Only these
// take the specialised kernels; the others run the general ones per group.
static bool dense(const ConvGeom& g) {
  return g.G == 1 && g.D == 1 && g.xs == (int64_t)g.C * g.HW && g.zs == (int64_t)g.OC * g.OHW;
}

// The geometry of one group of a grouped convolution (channel counts of the
// group, image strides of the whole tensors).
static ConvGeom group_geom(const ConvGeom& g) {
  ConvGeom s = g;
  s.C = g.C / g.G;
  s.OC = g.OC / g.G;
  s.J = s.C * g.K * g.K;
  return s;
}

// Weight-gradient tile shapes: BM x BN (x BK) and the TileShape that realises them.
enum DwShape { DW_64x64 = 0, DW_32x32, DW_32x64, DW_64x32, DW_128x64, DW_64x128, DW_128x128, DW_NSHAPES };
static const int kDwCand[DW_NSHAPES][3] = {{64, 64, 32},  {32, 32, 128}, {32, 64, 64}, {64, 32, 64},
                                           {128, 64, 32}, {64, 128, 32}, {128, 128, 32}};

struct DwPlan {
  int shape, bm, bn, bk, tiles_m, tiles_n, splits, groups;
  int64_t k_chunk;
  int conv1x1;                // 1: conv1x1_dw_kernel
  int rows_tc;                // > 0: conv_dw3_rows with this strip width
  int strips, rchunks, rlen;  // its strips, row runs per (image, strip), rows per run
};

// Row-streaming 3x3 dW: strip widths compiled in, and when to use it.
static const int kDw3Tc[] = {104, 64, 52, 32, 26};

static bool dw3_fits(int S, int tc) {
  switch (tc) {
#define CBB_FIT(T) \
  case T: return S == 1 ? Dw3RowCfg<1, T>::FITS : Dw3RowCfg<2, T>::FITS;
    CBB_FIT(104)
    CBB_FIT(64)
    CBB_FIT(52)
    CBB_FIT(32)
    CBB_FIT(26)
#undef CBB_FIT
  }
  return false;
}

static bool plan_dw3_rows(const ConvGeom& g, DwPlan& p) {
  if (!(g.K == 3 && g.P == 1 && (g.S == 1 || g.S == 2) && g.C % 32 == 0 && g.OC % 64 == 0))
    return false;
  int best_tc = 0;
  int64_t best_pad = 0;
  for (int tc : kDw3Tc) {
    if (!dw3_fits(g.S, tc)) continue;
    const int64_t padded = ceil_div(g.OW, tc) * tc;
    if (best_tc == 0 || padded < best_pad) {  // first (widest) wins ties
      best_tc = tc;
      best_pad = padded;
    }
  }
  if (best_pad * 8 > (int64_t)g.OW * 9) return false;  // > 1/8 of the columns wasted
  p = DwPlan{};
  p.rows_tc = best_tc;
  p.strips = (int)ceil_div(g.OW, best_tc);
  const int64_t nblk = (int64_t)(g.OC / 64) * (g.C / 32);
  const int64_t base = (int64_t)g.N * p.strips * nblk;
  // about 256 work-groups (one resident per CU), at least 4 rows per run
  int64_t rch = std::max<int64_t>(1, std::min<int64_t>(ceil_div(256, base), g.OH / 4));
  p.rlen = (int)ceil_div(g.OH, rch);
  p.rchunks = (int)ceil_div(g.OH, p.rlen);
  p.splits = g.N * p.strips * p.rchunks;
  p.groups = p.splits > kReduceGroup ? (int)ceil_div(p.splits, kReduceGroup) : 0;
  return true;
}

static bool conv1x1_ok(const ConvGeom& g) {
  return g.K == 1 && g.S == 1 && g.P == 0 && g.HW % 4 == 0 && g.C % 4 == 0;
}

static DwPlan plan_dw(const ConvGeom& g) {
  DwPlan best{};
  // the row-streaming kernel also takes the groups of a grouped layer (undilated)
  if (g.D == 1 && plan_dw3_rows(g, best)) return best;
  // 1x1: conv1x1_dw_dma when the tensors are 16-byte aligned (it has its own plan and
  // workspace, conv1x1_dw_workspace); otherwise the general kernel on these 64x64 tiles
  if (dense(g) && conv1x1_ok(g)) {
    best.conv1x1 = 1;
    best.shape = DW_64x64;
    best.bm = best.bn = 64;
    best.bk = 32;
    best.tiles_m = (int)ceil_div(g.OC, 64);
    best.tiles_n = (int)ceil_div(g.J, 64);
    const int64_t tiles = (int64_t)best.tiles_m * best.tiles_n;
    const int64_t ktiles = ceil_div(g.Q, 32);
    int64_t splits = ceil_div(512, tiles);
    splits = std::min<int64_t>(splits, std::max<int64_t>(1, ktiles / 4));
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, 4096));
    const int64_t chunk = ceil_div(ktiles, splits) * 32;
    best.splits = (int)ceil_div(g.Q, chunk);
    best.k_chunk = chunk;
    best.groups = best.splits > kReduceGroup ? (int)ceil_div(best.splits, kReduceGroup) : 0;
    return best;
  }
  double best_cost = 1e300;
  for (int s = 0; s < DW_NSHAPES; ++s) {
    const int bm = kDwCand[s][0], bn = kDwCand[s][1];
    const double tm = (double)ceil_div(g.OC, bm), tn = (double)ceil_div(g.J, bn);
    // padded matrix-core work, weighted by how well the tile shape feeds the
    // matrix cores (bigger wave tiles re-read LDS less per instruction)
    // measured on MI355X: 64x64 is the sweet spot; larger tiles did not pay off
    const double eff = (bm * bn > 64 * 64) ? 1.3 : (bm * bn == 64 * 64 ? 1.0 : 1.15);
    const double cost = tm * bm * tn * bn * eff;
    if (cost < best_cost) {
      best_cost = cost;
      best.shape = s;
      best.bm = bm;
      best.bn = bn;
      best.bk = kDwCand[s][2];
    }
  }
  best.tiles_m = (int)ceil_div(g.OC, best.bm);
  best.tiles_n = (int)ceil_div(g.J, best.bn);
  const int64_t tiles = (int64_t)best.tiles_m * best.tiles_n;
  const int64_t ktiles = ceil_div(g.Q, best.bk);
  const int64_t target = 1024;  // work-groups
  int64_t splits = ceil_div(target, tiles);
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, ktiles / 4));  // >= 4 K tiles each
  splits = std::max<int64_t>(1, std::min<int64_t>(splits, 4096));
  int64_t chunk = ceil_div(ktiles, splits) * best.bk;
  best.splits = (int)ceil_div(g.Q, chunk);
  best.k_chunk = chunk;
  best.groups = best.splits > kReduceGroup ? (int)ceil_div(best.splits, kReduceGroup) : 0;
  return best;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Fused small-channel dW + dX: which layers, and how the tiles are split.
bool conv_fused_dwdx_ok(const ConvGeom& g) {
  return dense(g) && g.C >= 1 && g.C <= 3 && g.K == 3 && g.P == 1 && g.S == 1 && g.OC <= 32 && g.W % 4 == 0;
}

struct FuPlan {
  int nstrips, sw, nruns, rlen, wgs, groups;
};

static FuPlan plan_fused(const ConvGeom& g, bool form_dz = false) {
  FuPlan p{};
  // strips of at most kFrMaxW columns, a multiple of 4, as even as possible
  const int ns0 = (int)ceil_div(g.W, kFrMaxW);
  p.sw = (int)(ceil_div(ceil_div(g.W, ns0), 4) * 4);
  p.nstrips = (int)ceil_div(g.W, p.sw);
  // runs of rows: about three work-groups per CU (two when dz is formed in the
  // kernel: its registers allow two per CU), at least 4 rows each (each run also
  // walks the dz rows just above and below it, so longer runs fetch less)
  const int64_t target = form_dz ? 512 : 768;
  int64_t runs = std::max<int64_t>(
      1, std::min<int64_t>(ceil_div(g.H, 4), ceil_div(target, (int64_t)g.N * p.nstrips)));
  // small layers (fewer than 64 work-groups that way): shorter runs, as many as keep
  // one level of the ordered dW sum (32 work-groups); the single 3x3 block (2 x 32 x
  // 32) measured 19 us on 16 four-row runs
  const int64_t cols = (int64_t)g.N * p.nstrips;
  if (cols * runs < 64 && cols < kReduceGroup)
    runs = std::max<int64_t>(runs, std::min<int64_t>(g.H, kReduceGroup / cols));
  p.rlen = (int)ceil_div(g.H, runs);
  p.nruns = (int)ceil_div(g.H, p.rlen);
  p.wgs = g.N * p.nstrips * p.nruns;
  p.groups = p.wgs > kReduceGroup ? (int)ceil_div(p.wgs, kReduceGroup) : 0;
  return p;
}

size_t conv_fused_workspace(const ConvGeom& g) {
  if (!conv_fused_dwdx_ok(g)) return 0;
  const FuPlan p = plan_fused(g), q = plan_fused(g, true);
  return ((size_t)std::max(p.wgs + p.groups, q.wgs + q.groups)) * g.OC * g.J * sizeof(float);
}


template <int CI>
static void launch_first_rows(const ConvGeom& g, const FuPlan& p, const float* x, const float* wt,
                              const float* dz, float* ws, float* dx, int accumulate,
                              const DzSource* src, hipStream_t st) {
  const DzSource s = src ? *src : DzSource{};
#define CBB_FR(FZ_)                                                                           \
  if (accumulate)                                                                             \
    conv_first_rows<CI, true, FZ_><<<p.wgs, kFrThreads, 0, st>>>(g, x, wt, dz, ws, dx,          \
                                                                 p.nstrips, p.sw, p.nruns,    \
                                                                 p.rlen, s);                  \
  else                                                                                        \
    conv_first_rows<CI, false, FZ_><<<p.wgs, kFrThreads, 0, st>>>(g, x, wt, dz, ws, dx,         \
                                                                  p.nstrips, p.sw, p.nruns,   \
                                                                  p.rlen, s)
  if (!src) {
    CBB_FR(kFzOff);
  } else {
    switch (src->y ? src->act : CBB_ACT_LINEAR) {
      case CBB_ACT_LINEAR: CBB_FR(CBB_ACT_LINEAR); break;
      case CBB_ACT_LEAKY: CBB_FR(CBB_ACT_LEAKY); break;
      case CBB_ACT_LOGISTIC: CBB_FR(CBB_ACT_LOGISTIC); break;
      case CBB_ACT_RELU: CBB_FR(CBB_ACT_RELU); break;
      default: CBB_FR(kFzAny); break;
    }
  }
#undef CBB_FR
}

int launch_conv_fused_dwdx(const ConvGeom& g, const float* x, const float* wt, const float* dz,
                           float* dw, float* dx, int accumulate, float* ws, hipStream_t st,
                           const DzSource* src) {
  const FuPlan p = plan_fused(g, src != nullptr);
  switch (g.C) {
    case 1: launch_first_rows<1>(g, p, x, wt, dz, ws, dx, accumulate, src, st); break;
    case 2: launch_first_rows<2>(g, p, x, wt, dz, ws, dx, accumulate, src, st); break;
    default: launch_first_rows<3>(g, p, x, wt, dz, ws, dx, accumulate, src, st); break;
  }
  const int rc = check_launch("conv_first_rows", st);
  if (rc) return rc;
  return launch_dw_reduce(g, dw, ws, p.wgs, p.groups, 0, st);
}

size_t conv_dw_workspace(const ConvGeom& g) {
  if (conv_depthwise(g)) return conv_depthwise_workspace(g);
  if (!dense(g)) {   // a partial region per group
    const ConvGeom s = group_geom(g);
    const DwPlan p = plan_dw(s);
    return p.splits == 1 ? 0
                         : (size_t)g.G * ((size_t)p.splits + p.groups) * s.OC * s.J * sizeof(float);
  }
  const DwPlan p = plan_dw(g);
  const size_t c1 = p.conv1x1 ? conv1x1_dw_workspace(g) : 0;
  if (p.splits == 1) return c1;
  const size_t mn = (size_t)g.OC * g.J;
  return std::max(c1, ((size_t)p.splits + p.groups) * mn * sizeof(float));
}

template <class TS>
static void launch_dw_tile(const ConvGeom& g, const DwPlan& p, const float* x, const float* dz,
                           float* out, int direct, hipStream_t st) {
  // grouped: one grid row per group; its output is its dW block, or its partial region
  const int64_t mn = (int64_t)g.OC * g.J;
  const int64_t ostride = direct ? mn : ((int64_t)p.splits + p.groups) * mn;
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n * p.splits), (unsigned)g.G);
  conv_dw_kernel<TS><<<grid, kThreads, 0, st>>>(g, x, dz, out, p.k_chunk, p.tiles_n, p.splits,
                                                direct, ostride);
}

// Grouped layers (g the group geometry): all groups in one launch on the grid's y
// axis; group j's dW block (direct) or partial region is out_gstride floats on.
template <int S>
static void launch_dw3_rows(const ConvGeom& g, const DwPlan& p, const float* x, const float* dz,
                            float* out, int direct, hipStream_t st, const DzSource* src = nullptr,
                            float* dzout = nullptr) {
  const int64_t mn = (int64_t)g.OC * g.J;
  const int64_t out_gstride = direct ? g.gw : ((int64_t)p.splits + p.groups) * mn;
  const unsigned blocks = (unsigned)((int64_t)p.splits * (g.OC / 64) * (g.C / 32));
  // 16-byte loads: rows and strip origins on 16-byte boundaries
  const bool v4 = aligned16(x) && aligned16(dz) && g.W % 4 == 0 && g.OW % 4 == 0 &&
                  p.rows_tc % 4 == 0;
  const DzSource s = src ? *src : DzSource{};
#define CBB_DW3K(TC, V4, FZ)                                                                 \
  conv_dw3_rows<S, TC, V4, FZ><<<dim3(blocks, (unsigned)g.G), kDw3Threads, 0, st>>>(        \
      g, x, dz, out, p.strips, p.rchunks, p.rlen, direct, s, dzout, out_gstride)
#define CBB_DW3(TC)                                                                          \
  case TC:                                                                                   \
    if constexpr (Dw3RowCfg<S, TC>::FITS) {                                                  \
      if (src && !src->y) /* no activation: y is never read */                            \
        CBB_DW3K(TC, true, CBB_ACT_LINEAR);                                                  \
      else if (src && src->act == CBB_ACT_LEAKY)                                             \
        CBB_DW3K(TC, true, CBB_ACT_LEAKY);                                                   \
      else if (src)                                                                          \
        CBB_DW3K(TC, true, kFzAny);                                                          \
      else if (v4)                                                                           \
        CBB_DW3K(TC, true, kFzOff);                                                          \
      else                                                                                   \
        CBB_DW3K(TC, false, kFzOff);                                                         \
    }                                                                                        \
    break;
  switch (p.rows_tc) {
    CBB_DW3(104)
    CBB_DW3(64)
    CBB_DW3(52)
    CBB_DW3(32)
    default:
      CBB_DW3K(26, false, kFzOff);
  }
#undef CBB_DW3
#undef CBB_DW3K
}

// Whether the weight gradient of this layer can form dz itself (conv_dw3_rows on its
// 16-byte path) from delta, y and x_norm, writing it to dz for the input gradient.
// Only with one block of 32 input channels: every input-channel block stages the dz
// rows again, and with four blocks (the 128-channel residual layer) the three
// tensors' extra loads cost more (147 against 120 + 20 µs) than the pass they save;
// with one (the stem's second layer) the stage drops from 476 to 445 µs.
bool conv_dw_forms_dz_ok(const ConvGeom& g) {
  if (!dense(g) || g.C != 32) return false;
  DwPlan p{};
  return plan_dw3_rows(g, p) && p.rows_tc % 4 == 0 && g.W % 4 == 0 && g.OW % 4 == 0;
}

// dW with dz formed inside the kernel from delta (and src), dz written to dzout.
// The caller has checked conv_dw_forms_dz_ok and the 16-byte alignment of every tensor.
int launch_conv_dw_forming_dz(const ConvGeom& g, const float* x, const float* delta,
                              const DzSource& src, float* dzout, float* dw, float* ws,
                              hipStream_t st) {
  DwPlan p{};
  if (!conv_dw_forms_dz_ok(g) || !plan_dw3_rows(g, p)) return CBB_EUNSUPPORTED;
  // the kernel reads y for every activation but LINEAR (selected when y is NULL)
  if (!src.coef || !dzout || (src.y == nullptr && src.act != CBB_ACT_LINEAR)) return CBB_EINVAL;
  const int direct = p.splits == 1;
  float* out = direct ? dw : ws;
  if (g.S == 1)
    launch_dw3_rows<1>(g, p, x, delta, out, direct, st, &src, dzout);
  else
    launch_dw3_rows<2>(g, p, x, delta, out, direct, st, &src, dzout);
  const int rc = check_launch("conv_dw3_rows (dz formed)", st);
  if (rc != CBB_OK || direct) return rc;
  return launch_dw_reduce(g, dw, ws, p.splits, p.groups, 1, st);
}

// dW of one group (or of a plain convolution).
static int launch_conv_dw_plain(const ConvGeom& g, const float* x, const float* dz, float* dw,
                                float* ws, hipStream_t st) {
  const DwPlan p = plan_dw(g);
  const int direct = p.splits == 1;
  float* out = direct ? dw : ws;
  if (p.conv1x1 && conv1x1_dma_ok(g, x, dz)) return launch_conv1x1_dw(g, x, dz, dw, ws, st);
  if (p.conv1x1) {
    // the direct copies need 16-byte aligned tensors; otherwise the general kernel
    // runs 64 x 64 tiles with the same split over K
    launch_dw_tile<TileShape<2, 2, 1>>(g, p, x, dz, out, direct, st);
  } else if (p.rows_tc > 0) {
    if (g.S == 1)
      launch_dw3_rows<1>(g, p, x, dz, out, direct, st);
    else
      launch_dw3_rows<2>(g, p, x, dz, out, direct, st);
  } else
  switch (p.shape) {
    case DW_64x64: launch_dw_tile<TileShape<2, 2, 1>>(g, p, x, dz, out, direct, st); break;
    case DW_32x32: launch_dw_tile<TileShape<1, 1, 4>>(g, p, x, dz, out, direct, st); break;
    case DW_32x64: launch_dw_tile<TileShape<1, 2, 2>>(g, p, x, dz, out, direct, st); break;
    case DW_64x32: launch_dw_tile<TileShape<2, 1, 2>>(g, p, x, dz, out, direct, st); break;
    case DW_128x64: launch_dw_tile<TileShape<2, 2, 1, 1, 2, 1>>(g, p, x, dz, out, direct, st); break;
    case DW_64x128: launch_dw_tile<TileShape<2, 2, 1, 1, 1, 2>>(g, p, x, dz, out, direct, st); break;
    default: launch_dw_tile<TileShape<2, 2, 1, 1, 2, 2>>(g, p, x, dz, out, direct, st); break;
  }
  int rc = check_launch(p.rows_tc > 0 ? "conv_dw3_rows" : "conv_dw_kernel", st);
  if (rc != CBB_OK || direct) return rc;
  return launch_dw_reduce(g, dw, ws, p.splits, p.groups, p.rows_tc > 0, st);
}

int launch_conv_dw(const ConvGeom& g, const float* x, const float* dz, float* dw, float* ws,
                   hipStream_t st) {
  if (conv_depthwise(g)) return launch_depthwise_dw(g, x, dz, dw, ws, st);
  // grouped or dilated: the general kernel on the group geometry, all groups in one
  // launch (group j: input channels j*C/G.., output channels j*OC/G.., weight block j)
  return launch_conv_dw_plain(dense(g) ? g : group_geom(g), x, dz, dw, ws, st);
}

// dw += ordered sum of the `splits` partials in ws (two levels when groups > 0).
int launch_dw_reduce(const ConvGeom& g, float* dw, float* ws, int splits, int groups,
                     int tapmajor, hipStream_t st) {
  const int64_t mn = (int64_t)g.OC * g.J;
  // 16-byte pieces of the partials when each region stays 16-byte aligned (ws is) and
  // there are enough of them (on small layers the scalar form, with 4x the threads,
  // measured faster)
  const bool v4 = mn % 4 == 0 && aligned16(ws) && mn >= kRedVecMin;
  const unsigned eblocks = (unsigned)ceil_div(v4 ? mn / 4 : mn, kThreads);
  const int kk = tapmajor ? g.K * g.K : 0;
  // grouped convolution: grid z = group, each with its own partial region
  const int64_t region = ((int64_t)splits + groups) * mn;
  // the last level: dW order, or the tap-major partials regrouped (9 taps)
  auto last = [&](const float* part, int n) -> int {
    if (kk == 9) {
      dw_reduce_tap<<<dim3((unsigned)ceil_div(g.C, 64), (unsigned)g.OC, g.G), kTapRedThreads, 0,
                      st>>>(dw, part, n, mn, g.OC, g.C, region);
      return check_launch("dw_reduce_l2", st);
    }
    if (kk != 0) return CBB_EUNSUPPORTED;
    const bool w4 = v4 && aligned16(dw);   // 16-byte adds into dW too
    const unsigned b2 = (unsigned)ceil_div(w4 ? mn / 4 : mn, kThreads);
    if (w4)
      dw_reduce_l2<4><<<dim3(b2, 1, g.G), kThreads, 0, st>>>(dw, part, n, mn, region);
    else
      dw_reduce_l2<1><<<dim3(b2, 1, g.G), kThreads, 0, st>>>(dw, part, n, mn, region);
    return check_launch("dw_reduce_l2", st);
  };
  if (groups == 0) return last(ws, splits);
  float* part2 = ws + (int64_t)splits * mn;
  if (v4)
    dw_reduce_l1<4><<<dim3(eblocks, groups, g.G), kThreads, 0, st>>>(ws, part2, splits, mn,
                                                                     region);
  else
    dw_reduce_l1<1><<<dim3(eblocks, groups, g.G), kThreads, 0, st>>>(ws, part2, splits, mn,
                                                                     region);
  const int rc = check_launch("dw_reduce_l1", st);
  if (rc) return rc;
  return last(part2, groups);
}

// ----------------------------------------------------------------------------- dX planning
enum DxKind { DX_SMALLC = 0, DX_32x128, DX_64x64, DX_D3S1, DX_D3S2, DX_1X1, DX_D3S1_SMALL, DX_COL };

// The column-buffer route (below) for small layers: its buffer, N x C k^2 x OH OW floats.
constexpr int64_t kColMaxBytes = int64_t(32) << 20;
static int64_t col_bytes(const ConvGeom& g) { return (int64_t)g.N * g.J * g.OHW * 4; }

struct DxPlan {
  int kind, bm, bn, bk, ctiles, pixtiles, ksplits;
};

static bool smallc_ok(const ConvGeom& g) {
  return g.C <= 4 && g.S == 1 && (g.K == 1 || g.K == 3 || g.K == 5 || g.K == 7);
}

static DxPlan plan_dx(const ConvGeom& g) {
  DxPlan p{};
  const bool special = dense(g);   // the specialised kernels assume a plain convolution
  // the tile-direct 3x3 kernels also take the groups of a grouped convolution (g is
  // then the group geometry; one grid row per group)
  const bool tile3 = special || (g.G > 1 && g.D == 1);
  // stride-1 tile-direct: the plain or grouped 3x3 pad-1 layers, and ungrouped 3x3
  // layers at dilation 2 with pad 2 (the same output size)
  const bool s1_direct =
      g.K == 3 && g.S == 1 &&
      ((tile3 && g.P == 1 && g.D == 1) ||
       (g.G == 1 && g.D == 2 && g.P == 2 && g.xs == (int64_t)g.C * g.HW &&
        g.zs == (int64_t)g.OC * g.OHW));
  if (special && smallc_ok(g)) {
    p.kind = DX_SMALLC;
    p.ksplits = 1;
    return p;
  }
  if (special && conv1x1_ok(g)) {
    p.kind = DX_1X1;
    p.ksplits = 1;
    p.ctiles = (int)ceil_div(g.C, 64);
    p.pixtiles = (int)ceil_div(g.Q, 64);
    return p;
  }
  // tile-direct 3x3: split the output channels when the grid cannot fill the GPU, as
  // many splits as fit one round of resident work-groups (`per_cu` of them on each of
  // the 256 CUs: a partial second round leaves most CUs idle while it runs), keeping
  // >= 4 chunks per split.  Measured on MI355X on the 26x26 head (96 blocks, two per
  // CU): 5 splits (480 work-groups) 139 + 9 us for the split sum, 11 splits (1056)
  // 150 + 14 us, 16 splits 147 + 18 us
  auto direct_splits = [&](int64_t blocks, int nchunks, int per_cu) {
    int64_t ks = std::max<int64_t>(1, 256 * per_cu / blocks);
    ks = std::min<int64_t>(ks, std::max<int64_t>(1, nchunks / 4));
    return (int)std::min<int64_t>(ks, 16);
  };
  // stride 1: larger images (>= 1024 pixels per plane) measured faster with the
  // small (128-pixel, 32-channel) tile, smaller ones with the 256-pixel, 64-channel tile
  if (s1_direct && (int64_t)g.H * g.W >= 1024 &&
      dx3_s1_fits(g.W, 1, Dx3Cfg<1, 1, 1>::ZPLANE, g.D) && g.C % Dx3Cfg<1, 1, 1>::BMC == 0 &&
      g.OC % Dx3Cfg<1, 1, 1>::OCB == 0) {
    using Cf = Dx3Cfg<1, 1, 1>;
    p.kind = DX_D3S1_SMALL;
    p.pixtiles = (int)ceil_div((int64_t)g.H * g.W, 128);
    p.ctiles = g.C / Cf::BMC;
    p.ksplits = direct_splits((int64_t)g.N * p.pixtiles * p.ctiles * g.G, g.OC / Cf::OCB, 3);
    return p;
  }
  if (s1_direct && dx3_s1_fits(g.W, 2, Dx3Cfg<1, 2, 2>::ZPLANE, g.D) &&
      g.C % Dx3Cfg<1, 2, 2>::BMC == 0 && g.OC % Dx3Cfg<1, 2, 2>::OCB == 0) {
    using Cf = Dx3Cfg<1, 2, 2>;
    p.kind = DX_D3S1;
    p.pixtiles = (int)ceil_div((int64_t)g.H * g.W, 128 * 2);
    p.ctiles = g.C / Cf::BMC;
    p.ksplits = direct_splits((int64_t)g.N * p.pixtiles * p.ctiles * g.G, g.OC / Cf::OCB, 2);
    return p;
  }
  if (tile3 && g.K == 3 && g.P == 1 && g.S == 2 && g.C % Dx3Cfg<2, 1, 1>::BMC == 0 &&
      g.OC % Dx3Cfg<2, 1, 1>::OCB == 0) {
    using Cf = Dx3Cfg<2, 1, 1>;
    p.kind = DX_D3S2;
    p.pixtiles = (int)(ceil_div(g.H, 8) * ceil_div(g.W, 64));
    p.ctiles = g.C / Cf::BMC;
    p.ksplits = direct_splits((int64_t)g.N * p.pixtiles * p.ctiles * g.G, g.OC / Cf::OCB, 2);
    return p;
  }
  // small layers with a 4x4 or larger window: the column buffer (a batched matrix-core
  // GEMM, then a gather of k^2 entries per element) beats the implicit GEMM, whose
  // index work per gathered element dominates at these sizes
  if (special && g.K >= 4 && g.OHW <= 1024 && col_bytes(g) <= kColMaxBytes) {
    p.kind = DX_COL;
    p.ksplits = 1;
    return p;
  }
  const int S = g.S;
  const int64_t maxpix = (int64_t)g.N * ((g.H + S - 1) / S) * ((g.W + S - 1) / S);
  p.bk = 32;
  // Measured on MI355X: one 32x32 block per wave beats larger wave tiles here (the
  // gathers, not the matrix cores, set the pace).
  if (g.C <= 32) {
    p.kind = DX_32x128; p.bm = 32; p.bn = 128;
  } else {
    p.kind = DX_64x64; p.bm = 64; p.bn = 64;
  }
  p.ctiles = (int)ceil_div(g.C, p.bm);
  p.pixtiles = (int)ceil_div(maxpix, p.bn);
  const int64_t blocks = (int64_t)p.ctiles * p.pixtiles * S * S;
  // average K per phase, in tiles
  const int64_t ocp = ceil_div(g.OC, p.bk) * p.bk;
  const int64_t ktiles = std::max<int64_t>(1, ceil_div(ocp * g.K * g.K / (S * S), p.bk));
  const int64_t target = 2048;   // work-groups in flight
  int64_t ks = ceil_div(target, blocks);
  ks = std::min<int64_t>(ks, std::max<int64_t>(1, ktiles / 4));  // >= 4 K tiles each
  p.ksplits = (int)std::max<int64_t>(1, std::min<int64_t>(ks, 16));
  return p;
}

bool conv_dx_sums_below_ok(const ConvGeom& g) {
  if (!dense(g)) return false;
  const DxPlan p = plan_dx(g);
  return p.kind == DX_D3S2 && p.ksplits == 1 && (g.OC == 64 || g.OC == 128) && p.ctiles == 1 &&
         g.OW % 4 == 0 && g.W % 4 == 0;
}

// 1 when launch_conv_dx runs a specialised kernel for g (tile-direct 3x3 or the 1x1
// copy ring), not the general one.
bool conv_dx_specialised(const ConvGeom& g) {
  if (!dense(g)) return false;
  const DxPlan p = plan_dx(g);
  return p.kind == DX_D3S1 || p.kind == DX_D3S1_SMALL || p.kind == DX_D3S2 || p.kind == DX_1X1;
}

size_t conv_dx_workspace(const ConvGeom& g) {
  if (conv_depthwise(g)) return 0;
  // grouped: every group writes its channels of the same [split][n][c][hw] partials
  const DxPlan p = plan_dx(dense(g) ? g : group_geom(g));
  if (p.kind == DX_COL) return (size_t)col_bytes(g);
  if (p.ksplits <= 1) return 0;
  return (size_t)p.ksplits * g.N * g.C * g.HW * sizeof(float);
}

template <int CI>
static void launch_smallc(const ConvGeom& g, const float* wt, const float* dz, float* dx,
                          int accumulate, hipStream_t st) {
  const int tiles_w = (int)ceil_div(g.W, kScTW), tiles_h = (int)ceil_div(g.H, kScTH);
  const unsigned blocks = (unsigned)(g.N * tiles_w * tiles_h);
  switch (g.K) {
    case 1: conv_dx_smallc_kernel<CI, 1><<<blocks, kThreads, 0, st>>>(g, wt, dz, dx, tiles_w, tiles_h, accumulate); break;
    case 3: conv_dx_smallc_kernel<CI, 3><<<blocks, kThreads, 0, st>>>(g, wt, dz, dx, tiles_w, tiles_h, accumulate); break;
    case 5: conv_dx_smallc_kernel<CI, 5><<<blocks, kThreads, 0, st>>>(g, wt, dz, dx, tiles_w, tiles_h, accumulate); break;
    default: conv_dx_smallc_kernel<CI, 7><<<blocks, kThreads, 0, st>>>(g, wt, dz, dx, tiles_w, tiles_h, accumulate); break;
  }
}

template <class TS>
static void launch_dx_mfma(const ConvGeom& g, const DxPlan& p, const float* wt, const float* dz,
                           float* dx, float* ws, int accumulate, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)p.pixtiles * g.S * g.S * p.ksplits * p.ctiles),
                  (unsigned)g.G);   // grouped: one grid row per group
  conv_dx_kernel<TS><<<grid, kThreads, 0, st>>>(g, wt, dz, dx, ws, p.ctiles, p.ksplits,
                                                p.pixtiles, accumulate);
}

int launch_conv_dx(const ConvGeom& g, const float* wt, const float* dz, float* dx, int accumulate,
                   float* ws, hipStream_t st, BnBelow* below) {
  if (below) below->nseg = 0;
  if (conv_depthwise(g)) return launch_depthwise_dx(g, wt, dz, dx, accumulate, st);
  // the tile-direct 3x3 kernel over g (a plain layer, or the group geometry of a
  // grouped one: one grid row per group), then the ordered sum of the split partials
  auto tile_direct = [&](const ConvGeom& t, const DxPlan& p) {
    const unsigned blocks = (unsigned)((int64_t)t.N * p.pixtiles * p.ctiles * p.ksplits);
    const dim3 grid(blocks, (unsigned)t.G);
    const int tiles_w = p.kind == DX_D3S2 ? (int)ceil_div(t.W, 64) : 0;
    // 16-byte copies need every group's weights and dz 16-byte aligned too
    const bool wal = aligned16(wt) && (t.G == 1 || t.gw % 4 == 0);
    // 16-byte tile copies: the tile rows (W + 8 floats) must still fit the plane
    const int f1 = p.kind == DX_D3S1 ? 2 : 1;
    const bool z4 = wal && aligned16(dz) && (t.G == 1 || t.gz % 4 == 0) &&
                    (t.S == 1 ? t.W % 4 == 0 && t.D <= 4 &&
                                    ((128 * f1 - 1) / t.W + 2 + 2 * t.D) * (t.W + 8) <=
                                        Dx3Cfg<1, 1, 1>::ZPLANE
                              : t.OW % 4 == 0);
#define CBB_DX3D(S_, F_, RM_, Z4_, DIL_)                                                  \
  if (wal)                                                                                \
    conv_dx3_direct<S_, F_, RM_, true, Z4_, DIL_><<<grid, kThreads, 0, st>>>(             \
        t, wt, dz, dx, ws, accumulate, p.pixtiles, tiles_w, p.ksplits);                   \
  else                                                                                    \
    conv_dx3_direct<S_, F_, RM_, false, false, DIL_><<<grid, kThreads, 0, st>>>(          \
        t, wt, dz, dx, ws, accumulate, p.pixtiles, tiles_w, p.ksplits);
#define CBB_DX3(S_, F_, RM_, Z4_) CBB_DX3D(S_, F_, RM_, Z4_, 1)
    if (p.kind == DX_D3S1) {
      if (t.D == 2) {
        if (z4) {
          CBB_DX3D(1, 2, 2, true, 2)
        } else {
          CBB_DX3D(1, 2, 2, false, 2)
        }
      } else if (z4) {
        CBB_DX3(1, 2, 2, true)
      } else {
        CBB_DX3(1, 2, 2, false)
      }
    } else if (p.kind == DX_D3S1_SMALL) {
      if (t.D == 2) {
        if (z4) {
          CBB_DX3D(1, 1, 1, true, 2)
        } else {
          CBB_DX3D(1, 1, 1, false, 2)
        }
      } else if (z4) {
        CBB_DX3(1, 1, 1, true)
      } else {
        CBB_DX3(1, 1, 1, false)
      }
    } else {
      if (z4) {
        CBB_DX3(2, 1, 1, true)
      } else {
        CBB_DX3(2, 1, 1, false)
      }
    }
#undef CBB_DX3
#undef CBB_DX3D
    int rc = check_launch("conv_dx3_direct", st);
    if (rc || p.ksplits == 1) return rc;
    return launch_dx_reduce(dx, ws, p.ksplits, (int64_t)g.N * g.C * g.HW, accumulate, st);
  };
  auto is_tile3 = [](const DxPlan& p) {
    return p.kind == DX_D3S1 || p.kind == DX_D3S1_SMALL || p.kind == DX_D3S2;
  };
  if (!dense(g)) {
    const ConvGeom s = group_geom(g);
    const DxPlan p = plan_dx(s);
    // grouped, undilated 3x3 pad 1 (all groups in one launch), or dilated 3x3 with pad
    // equal to the dilation: the tile-direct kernel
    if (is_tile3(p)) return tile_direct(s, p);
    // grouped or dilated otherwise: the general kernel on the group geometry, all
    // groups in one launch (group j: input channels j*C/G.., output channels
    // j*OC/G.., weight block j), then one ordered sum of the split partials over all
    // channels
    if (p.kind == DX_32x128)
      launch_dx_mfma<TileShape<1, 4, 1>>(s, p, wt, dz, dx, p.ksplits > 1 ? ws : nullptr,
                                         accumulate, st);
    else
      launch_dx_mfma<TileShape<2, 2, 1>>(s, p, wt, dz, dx, p.ksplits > 1 ? ws : nullptr,
                                         accumulate, st);
    const int rc = check_launch("conv_dx_kernel", st);
    if (rc || p.ksplits == 1) return rc;
    return launch_dx_reduce(dx, ws, p.ksplits, (int64_t)g.N * g.C * g.HW, accumulate, st);
  }
  const DxPlan p = plan_dx(g);
  if (is_tile3(p)) {
    const int tiles_w = p.kind == DX_D3S2 ? (int)ceil_div(g.W, 64) : 0;
    if (p.kind == DX_D3S2 && aligned16(wt) && aligned16(dz) && g.OW % 4 == 0 &&
        p.ksplits == 1 && (g.OC == 64 || g.OC == 128)) {
      const int ntiles = (int)((int64_t)g.N * p.pixtiles * p.ctiles);
      const unsigned grid = (unsigned)std::min(ntiles, kDxS2pGroups);
      // the block below's act/BN sums in the epilogue: one 32-channel tile column
      // (a work-group's tiles then all hold the same channels) and whole 16-byte rows
      const bool sums = below && below->part && below->xn && p.ctiles == 1 &&
                        g.W % 4 == 0 && aligned16(dx) && aligned16(below->xn) &&
                        (!below->y || aligned16(below->y));
      BnBelow ba{};
      if (sums) {
        ba = *below;
        if (!ba.y) ba.y = ba.xn;   // LINEAR: y is not read, any valid address will do
        below->nseg = (int)grid;
      }
#define CBB_S2P(NCH_, BA_)                                                                 \
  conv_dx3_s2p<NCH_, BA_><<<grid, kThreads, 0, st>>>(g, wt, dz, dx, accumulate, ntiles,  \
                                                     p.pixtiles, tiles_w, ba)
      if (!sums) {
        if (g.OC == 64) CBB_S2P(4, kFzOff); else CBB_S2P(8, kFzOff);
      } else if (ba.act == CBB_ACT_LEAKY) {
        if (g.OC == 64) CBB_S2P(4, CBB_ACT_LEAKY); else CBB_S2P(8, CBB_ACT_LEAKY);
      } else {
        if (g.OC == 64) CBB_S2P(4, kFzAny); else CBB_S2P(8, kFzAny);
      }
#undef CBB_S2P
      return check_launch(sums ? "conv_dx3_s2p (act/BN sums below)" : "conv_dx3_s2p", st);
    }
    return tile_direct(g, p);
  }
  if (p.kind == DX_1X1) {
    if (conv1x1_dma_ok(g, wt, dz)) return launch_conv1x1_dx(g, wt, dz, dx, accumulate, st);
    // misaligned tensors: the general kernel on 64 x 64 tiles, no split
    launch_dx_mfma<TileShape<2, 2, 1>>(g, p, wt, dz, dx, ws, accumulate, st);
    return check_launch("conv_dx_kernel", st);
  }
  if (p.kind == DX_COL) {
    // col[n][(i,kh,kw)][p] = sum_o W[o][i][kh][kw] dz[n][o][p], one GEMM per image
    GemmArgs ga{g.J, g.OHW, g.OC, wt, 1, g.J, dz, g.OHW, 1, ws, g.OHW, 0, g.zs,
                (int64_t)g.J * g.OHW};
    int rc = launch_gemm(ga, st, g.N);
    if (rc) return rc;
    const int64_t n = (int64_t)g.N * g.C * g.HW;
    const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(n, kThreads), 16384);
    if (g.S == 1)
      col2im_kernel<true><<<blocks, kThreads, 0, st>>>(g, ws, dx, accumulate);
    else
      col2im_kernel<false><<<blocks, kThreads, 0, st>>>(g, ws, dx, accumulate);
    return check_launch("conv_dx_col2im", st);
  }
  if (p.kind == DX_SMALLC) {
    switch (g.C) {
      case 1: launch_smallc<1>(g, wt, dz, dx, accumulate, st); break;
      case 2: launch_smallc<2>(g, wt, dz, dx, accumulate, st); break;
      case 3: launch_smallc<3>(g, wt, dz, dx, accumulate, st); break;
      default: launch_smallc<4>(g, wt, dz, dx, accumulate, st); break;
    }
    return check_launch("conv_dx_smallc_kernel", st);
  }
  if (p.kind == DX_32x128)
    launch_dx_mfma<TileShape<1, 4, 1>>(g, p, wt, dz, dx, ws, accumulate, st);
  else
    launch_dx_mfma<TileShape<2, 2, 1>>(g, p, wt, dz, dx, ws, accumulate, st);
  int rc = check_launch("conv_dx_kernel", st);
  if (rc || p.ksplits == 1) return rc;
  return launch_dx_reduce(dx, ws, p.ksplits, (int64_t)g.N * g.C * g.HW, accumulate, st);
}

}  // namespace cbb
