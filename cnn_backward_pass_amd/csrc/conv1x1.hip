// conv1x1.hip -- weight and input gradients of a 1x1, stride-1, unpadded
// convolution on the gfx950 fp32 matrix cores.
//
// Pages: "YOLOv3 backpropagation: full-flow source analysis" (suzhouguqin.com),
// section 3.1 (backward_convolutional_layer) with section 3.2's im2col at
// size 1, stride 1, pad 0, where the column matrix is the input itself.  The two
// gradients are then plain GEMMs over the pixels q = (n, p):
//   dW[o][i]    += sum_q dz[n][o][p] * x[n][i][p]      (M = o, N = i, K = q)
//   dx[n][i][p]  = sum_o W[o][i] * dz[n][o][p]         (M = i, N = q, K = o)
//
// Both kernels stage their operand tiles with direct global-to-LDS copies (16
// bytes per lane, no registers in between) into two LDS buffers, so the next K
// tile lands while the matrix cores work on this one.  H*W and C_in are
// multiples of 4 (checked on the host), so a 16-byte piece of a pixel row never
// straddles two images; pieces outside the matrices (ragged M, N or K) are
// copied from a zero page, which makes their products exactly zero.
//
// Work-group: 4 waves as 2 (M) x 2 (N); a wave owns (TM/2) x (TN/2) of the
// work-group tile as RM x RN blocks of 32 x 32, one v_mfma_f32_32x32x2_f32
// accumulator each.  K tiles are 32 deep.
#include "cbb_internal.h"

namespace cbb {

// Source of the padding copies (never written).
__device__ float g_c1_zero[4];

typedef float c1f4 __attribute__((ext_vector_type(4)));

// One direct global-to-LDS copy of 16 bytes per lane into the 1 KB at `lds`
// (lane l fills bytes 16 l .. 16 l + 15; M0 holds the LDS address).  Written as
// inline assembly so that the compiler does not track it: its own wait
// insertion cannot tell the ring buffers apart and would drain every copy in
// flight before each LDS read.  The kernels here wait with explicit counts
// (wait_vmem) before a buffer is read, nothing else in them uses M0, and no
// copy is in flight when a kernel ends.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const float* src, float* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)lds_ptr(lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(a)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// K loop over nk tiles with NS LDS buffers holding tiles t+1 .. t+NS while the
// matrix cores work on tile t from registers; the operands of tile t+1 are read
// from LDS into the other register set during that work, so the reads' latency
// and the LDS traffic of all waves overlap the matrix instructions.
//   issue(t, s): copy tile t into buffer s (PER copy instructions per wave, the
//                same for every tile)
//   fetch(s, r): read this wave's operands of buffer s into register set r
//   mma(r):      the matrix work on register set r
// Before fetching tile t+1: this wave's copies of it have landed (loads of one
// wave complete in order, so only the copies of later tiles may be outstanding)
// and its reads of tile t are complete; after the barrier the same holds for
// every wave, so tile t's buffer takes tile t + NS.
template <int NS, int PER, class Issue, class Fetch, class Mma>
__device__ __forceinline__ void dma_ring(int nk, Issue&& issue, Fetch&& fetch, Mma&& mma) {
  constexpr int U = NS % 2 == 0 ? NS : 2 * NS;   // buffer and register-set indices repeat
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nk) issue(s, s);
  if (nk <= 0) return;
  if (nk >= NS)
    wait_vmem<(NS - 1) * PER>();
  else
    wait_vmem<0>();
  // a bare barrier: __syncthreads() would also wait for every copy in flight
  asm volatile("s_barrier" ::: "memory");
  fetch(0, 0);
  for (int kt = 0; kt < nk; kt += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = kt + u;
      if (t < nk) {
        if (t + 1 < nk) {
          if (t + NS <= nk)
            wait_vmem<(NS - 2) * PER>();
          else
            wait_vmem<0>();
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          if (t + NS < nk) issue(t + NS, u % NS);
          fetch((u + 1) % NS, (u + 1) % 2);
        }
        mma(u % 2);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Input gradient.  LDS rows are K rows: A[k][m] = W[o0 + k][i0 + m] (TM floats)
// and B[k][n] = dz[.][o0 + k][pixel q0 + n] (TN floats), i.e. both operands keep
// their memory order.  A copy instruction of a wave fills 256 consecutive floats
// (256 / T rows).  Odd rows are stored rotated by 32 floats, so the two half-waves
// of an operand read (rows k and k + 1, same columns) use different LDS banks.
// No split over K: a work-group sums all output channels in a fixed order.
// ---------------------------------------------------------------------------
template <int TM, int TN, int NS>
__global__ __launch_bounds__(kThreads, 2) void conv1x1_dx_dma(ConvGeom g, const float* __restrict__ wt,
                                                           const float* __restrict__ dz,
                                                           float* __restrict__ dx, int mtiles,
                                                           int accumulate) {
  constexpr int BK = 32, RM = TM / 64, RN = TN / 64;
  constexpr int AI = BK * TM / 1024, BI = BK * TN / 1024;   // copies per wave per K tile
  // ring buffers, each picked by a compile-time index
  constexpr int AF = BK * TM, BF = BK * TN;
  __shared__ __attribute__((aligned(16))) float A0[AF], B0[BF], A1[AF], B1[BF];
  __shared__ __attribute__((aligned(16))) float A2[NS > 2 ? AF : 4], B2[NS > 2 ? BF : 4];
  __shared__ __attribute__((aligned(16))) float A3[NS > 3 ? AF : 4], B3[NS > 3 ? BF : 4];
  auto Ab = [&](int s) -> float* { return s == 0 ? A0 : s == 1 ? A1 : s == 2 ? A2 : A3; };
  auto Bb = [&](int s) -> float* { return s == 0 ? B0 : s == 1 ? B1 : s == 2 ? B2 : B3; };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1, col = lane & 31, hf = lane >> 5;
  // the M tiles of one pixel tile (same dz rows) run on one XCD, sharing its L2
  const int bid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int mt = bid % mtiles;
  const int i0 = mt * TM;
  const int64_t q0 = (int64_t)(bid / mtiles) * TN;

  // ---- copy sources.  Lane l fills floats 4l .. 4l+3 of a 256-float block: row
  // l / (T/4) of the block at physical column 4 (l % (T/4)), which holds logical
  // column (physical - 32 (row & 1)) mod T.  Blocks hold an even number of rows.
  constexpr int ALR = TM / 4, BLR = TN / 4;   // lanes per row
  const int arow = lane / ALR, brow = lane / BLR;
  const int acol = 4 * (((lane % ALR) - 8 * (arow & 1)) & (ALR - 1));
  const int bcol = 4 * (((lane % BLR) - 8 * (brow & 1)) & (BLR - 1));
  const bool aok = i0 + acol < g.C;
  const float* abase = wt + i0 + acol;                      // + o * C
  const int64_t qb = q0 + bcol;
  const bool bok = qb < g.Q;
  const int bn = bok ? (int)qb / g.HW : 0;
  const int bp = bok ? (int)qb - bn * g.HW : 0;
  const float* bbase = dz + (int64_t)bn * g.OC * g.HW + bp;  // + o * HW
  auto issue = [&](int t, int s) {
    const int o0 = t * BK;
    float* As = Ab(s);
    float* Bs = Bb(s);
#pragma unroll
    for (int r = 0; r < AI; ++r) {
      const int blk = wave + 4 * r;
      const int o = o0 + blk * (256 / TM) + arow;
      const float* src = (aok && o < g.OC) ? abase + (int64_t)o * g.C : g_c1_zero;
      dma16(src, As + 256 * blk);
    }
#pragma unroll
    for (int r = 0; r < BI; ++r) {
      const int blk = wave + 4 * r;
      const int o = o0 + blk * (256 / TN) + brow;
      const float* src = (bok && o < g.OC) ? bbase + (int64_t)o * g.HW : g_c1_zero;
      dma16(src, Bs + 256 * blk);
    }
  };

  // ---- operand reads: lane (col, hf) of K step s reads row 2s + hf
  int aoff[RM], boff[RN];
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    const int m = wm * (TM / 2) + i * 32 + col;
    aoff[i] = hf * TM + ((m + 32 * hf) & (TM - 1));
  }
#pragma unroll
  for (int j = 0; j < RN; ++j) {
    const int n = wn * (TN / 2) + j * 32 + col;
    boff[j] = hf * TN + ((n + 32 * hf) & (TN - 1));
  }
  f32x16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  float fa[2][16][RM], fb[2][16][RN];   // two register sets of a K tile's operands
  auto fetch = [&](int sb, int r) {
    const float* As = Ab(sb);
    const float* Bs = Bb(sb);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
#pragma unroll
      for (int i = 0; i < RM; ++i) fa[r][s][i] = As[aoff[i] + 2 * s * TM];
#pragma unroll
      for (int j = 0; j < RN; ++j) fb[r][s][j] = Bs[boff[j] + 2 * s * TN];
    }
  };
  auto mma = [&](int r) {
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[r][s][i], fb[r][s][j], acc[i][j], 0, 0, 0);
  };

  // ---- K loop over the output channels
  dma_ring<NS, AI + BI>((g.OC + BK - 1) / BK, issue, fetch, mma);

  // ---- epilogue: lane holds pixel q of column `col` of each block, channels acc_row(r)
  if (accumulate) {
    // every earlier value read (clamped addresses, so each load is issued) and added
    // before the first store: a wait for a load among the stores would also wait for
    // every store before it
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      const int64_t q = min(q0 + wn * (TN / 2) + j * 32 + col, g.Q - 1);
      const int n = (int)q / g.HW, p = (int)q - n * g.HW;
      const float* base = dx + (int64_t)n * g.C * g.HW + p;
#pragma unroll
      for (int i = 0; i < RM; ++i) {
        const int cb = i0 + wm * (TM / 2) + i * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[i][j][r] += base[(int64_t)min(cb + acc_row(r, lane), g.C - 1) * g.HW];
      }
    }
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(acc[i][j][r]));
  }
#pragma unroll
  for (int j = 0; j < RN; ++j) {
    const int64_t q = q0 + wn * (TN / 2) + j * 32 + col;
    if (q >= g.Q) continue;
    const int n = (int)q / g.HW, p = (int)q - n * g.HW;
    float* base = dx + (int64_t)n * g.C * g.HW + p;
#pragma unroll
    for (int i = 0; i < RM; ++i) {
      const int cb = i0 + wm * (TM / 2) + i * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = cb + acc_row(r, lane);
        if (c < g.C) base[(int64_t)c * g.HW] = acc[i][j][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Weight gradient.  A 64 x 64 block of dW per work-group of eight waves: wave
// (wm, wn, wk) owns the 32 x 32 quarter (wm, wn) and half wk of every K tile, so
// two waves share each SIMD and one's LDS reads, copy issue and barrier wait
// overlap the other's matrix work; the two K halves are summed through LDS at the
// end.  K tiles are 64 pixels q = (n, p) = k0 + k:
//   A[m][k] = dz[n][o0 + m][p],  B[m][k] = x[n][i0 + m][p]   (rows of 64 floats).
// A row is sixteen 16-byte pieces; piece c of row m sits at position c ^ (m & 15),
// so the 16-byte operand reads of 16 consecutive rows touch every LDS bank once.
// A copy instruction fills 4 rows (1 KB): lane l takes row l / 16 at position
// l % 16; over a wave's copies (blocks wave, wave + 8, ...) the row's low four
// bits, and so the piece, are the same.
// K order inside a tile: half wk holds pieces 8 wk .. 8 wk + 7; lane half hf of
// its step 4j + e multiplies the elements 4 (8 wk + 2j + hf) + e.  Both operands
// follow it, so the sum covers the tile's 64 pixels once.  Split over K:
// work-group (split, tile) sums the pixels [split * k_chunk, +k_chunk) and writes
// its partial block to out[split][o][i] (or adds into dW when there is one split).
// ---------------------------------------------------------------------------
constexpr int kC1DwThreads = 512;

template <int NS>
__global__ __launch_bounds__(kC1DwThreads, 1) void conv1x1_dw_dma(
    ConvGeom g, const float* __restrict__ x, const float* __restrict__ dz, float* __restrict__ out,
    int k_chunk, int mtiles, int ntiles, int direct) {
  constexpr int T = 64, BK = 64;
  constexpr int CI = T * BK / 256 / 8;   // copy instructions per wave per operand and K tile
  constexpr int F = T * BK;              // floats per operand and K tile
  __shared__ __attribute__((aligned(16))) float A0[F], B0[F], A1[F], B1[F];
  __shared__ __attribute__((aligned(16))) float A2[NS > 2 ? F : 4], B2[NS > 2 ? F : 4];
  auto Ab = [&](int s) -> float* { return s == 0 ? A0 : s == 1 ? A1 : A2; };
  auto Bb = [&](int s) -> float* { return s == 0 ? B0 : s == 1 ? B1 : B2; };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = (wave >> 1) & 1, wk = wave >> 2;
  const int col = lane & 31, hf = lane >> 5;
  const int tiles = mtiles * ntiles;
  // the tiles of one split (same pixels of dz and x) run on one XCD, sharing its L2
  const int bid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int split = bid / tiles, t = bid - split * tiles;
  const int o0 = (t % mtiles) * T, i0 = (t / mtiles) * T;
  const int kbeg = split * k_chunk;
  const int kend = (int)std::min<int64_t>(g.Q, (int64_t)kbeg + k_chunk);

  // ---- copy sources: row 4 blk + l / 16, piece (l % 16) ^ (row & 15)
  const int crow = lane >> 4;
  const int cpiece = (lane & 15) ^ ((4 * (wave & 3) + crow) & 15);
  auto issue = [&](int kt, int s) {
    float* As = Ab(s);
    float* Bs = Bb(s);
    const int q = kbeg + kt * BK + 4 * cpiece;
    const bool ok = q < kend;
    const int n = ok ? q / g.HW : 0, p = ok ? q - n * g.HW : 0;
    const float* ab = dz + ((int64_t)n * g.OC + o0) * g.HW + p;
    const float* bb = x + ((int64_t)n * g.C + i0) * g.HW + p;
#pragma unroll
    for (int r = 0; r < CI; ++r) {
      const int blk = wave + 8 * r, m = 4 * blk + crow;
      dma16((ok && o0 + m < g.OC) ? ab + (int64_t)m * g.HW : g_c1_zero, As + 256 * blk);
      dma16((ok && i0 + m < g.C) ? bb + (int64_t)m * g.HW : g_c1_zero, Bs + 256 * blk);
    }
  };

  // ---- operand reads: rows wm * 32 + col (A) and wn * 32 + col (B), pieces 8 wk + 2j + hf
  const int arow = (wm * 32 + col) * BK, brow = (wn * 32 + col) * BK;
  int po[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) po[j] = 4 * ((8 * wk + 2 * j + hf) ^ (col & 15));
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  c1f4 va[2][4], vb[2][4];   // two register sets of a K tile's operands
  auto fetch = [&](int sb, int r) {
    const float* As = Ab(sb);
    const float* Bs = Bb(sb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      va[r][j] = *(const c1f4*)(As + arow + po[j]);
      vb[r][j] = *(const c1f4*)(Bs + brow + po[j]);
    }
  };
  auto mma = [&](int r) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(va[r][j][e], vb[r][j][e], acc, 0, 0, 0);
  };

  dma_ring<NS, 2 * CI>((kend - kbeg + BK - 1) / BK, issue, fetch, mma);

  // ---- sum the two K halves (the ring's buffers are free: every copy has landed and
  // every wave is past its last read once all have reached the barrier)
  __syncthreads();
  float* red = A0;   // 4 waves x 16 x 64 floats
  if (wk == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) red[((wave & 3) * 16 + r) * 64 + lane] = acc[r];
  }
  __syncthreads();
  if (wk == 1) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] += red[((wave & 3) * 16 + r) * 64 + lane];

  float* dst = direct ? out : out + (int64_t)split * g.OC * g.C;
  const int c = i0 + wn * 32 + col;
  if (c >= g.C) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int o = o0 + wm * 32 + acc_row(r, lane);
    if (o < g.OC) {
      const int64_t e = (int64_t)o * g.C + c;
      if (direct)
        dst[e] += acc[r];
      else
        dst[e] = acc[r];
    }
  }
}

// ----------------------------------------------------------------------------- host side
bool conv1x1_dma_ok(const ConvGeom& g, const void* a, const void* b) {
  return g.K == 1 && g.S == 1 && g.P == 0 && g.HW % 4 == 0 && g.C % 4 == 0 &&
         g.Q < (int64_t)1 << 30 && ((uintptr_t)a & 15) == 0 && ((uintptr_t)b & 15) == 0;
}

// Tiles of 64 x 64 (measured on MI355X against 128 x 128, 128 x 64 and 64 x 128
// on the 1x1 layers of the YOLOv3 head and the Darknet-53 residual unit: within
// 10%, and 64 x 64 best or tied everywhere).  dX keeps three K tiles of 32 output
// channels in LDS, dW two of 64 pixels, with K split over at most 256 work-groups
// (one per CU: a few more would run as a second, short round).  Deeper rings, a
// second wave per SIMD and 512 work-groups measured no faster.
constexpr int kC1T = 64, kC1DxStages = 3, kC1DwStages = 2, kC1DwGroups = 256;

struct C1DwPlan {
  int mtiles, ntiles, splits, groups, k_chunk;
};

static C1DwPlan c1_plan_dw(const ConvGeom& g) {
  C1DwPlan p{};
  p.mtiles = (int)ceil_div(g.OC, kC1T);
  p.ntiles = (int)ceil_div(g.C, kC1T);
  const int64_t tiles = (int64_t)p.mtiles * p.ntiles, ktiles = ceil_div(g.Q, 64);
  // each split covers at least 4 K tiles of 64 pixels
  const int64_t splits = std::max<int64_t>(1, std::min<int64_t>(kC1DwGroups / tiles, ktiles / 4));
  p.k_chunk = (int)(ceil_div(ktiles, splits) * 64);
  p.splits = (int)ceil_div(g.Q, p.k_chunk);
  p.groups = p.splits > kReduceGroup ? (int)ceil_div(p.splits, kReduceGroup) : 0;
  return p;
}

size_t conv1x1_dw_workspace(const ConvGeom& g) {
  const C1DwPlan p = c1_plan_dw(g);
  if (p.splits == 1) return 0;
  return ((size_t)p.splits + p.groups) * g.OC * g.C * sizeof(float);
}

int launch_conv1x1_dw(const ConvGeom& g, const float* x, const float* dz, float* dw, float* ws,
                      hipStream_t st) {
  const C1DwPlan p = c1_plan_dw(g);
  const int direct = p.splits == 1;
  float* out = direct ? dw : ws;
  const unsigned blocks = (unsigned)((int64_t)p.mtiles * p.ntiles * p.splits);
  conv1x1_dw_dma<kC1DwStages><<<blocks, kC1DwThreads, 0, st>>>(g, x, dz, out, p.k_chunk,
                                                               p.mtiles, p.ntiles, direct);
  const int rc = check_launch("conv1x1_dw_dma", st);
  if (rc != CBB_OK || direct) return rc;
  return launch_dw_reduce(g, dw, ws, p.splits, p.groups, 0, st);
}

int launch_conv1x1_dx(const ConvGeom& g, const float* wt, const float* dz, float* dx,
                      int accumulate, hipStream_t st) {
  const int mtiles = (int)ceil_div(g.C, kC1T);
  const unsigned blocks = (unsigned)(mtiles * ceil_div(g.Q, kC1T));
  conv1x1_dx_dma<kC1T, kC1T, kC1DxStages><<<blocks, kThreads, 0, st>>>(g, wt, dz, dx, mtiles,
                                                                      accumulate);
  return check_launch("conv1x1_dx_dma", st);
}

}  // namespace cbb
