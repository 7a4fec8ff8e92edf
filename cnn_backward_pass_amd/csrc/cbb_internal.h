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

// Geometry of one convolution, derived from cbb_conv_desc.
struct ConvGeom {
  int N, C, H, W, OC, K, S, P, OH, OW;
  int HW, OHW, J;  // J = C*K*K, columns of the weight-gradient matrix
  int64_t Q;       // N*OH*OW, the reduction length of the weight gradient
};

// Host-side launch bookkeeping -------------------------------------------------
void set_hip_error(hipError_t e, const char* where);
int check_launch(const char* where);  // CBB_OK or CBB_EHIP after a launch

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
// wave owns a 32 x 32 output block (one 32x32x2 accumulator) and, when WK > 1,
// a quarter/half of every K tile, with the WK partial blocks summed through
// LDS at the end.  K tiles are BK = 32*WK deep and staged in LDS as
//   As[BK][BM + 1]  (A transposed: K-major, padded against bank conflicts)
//   Bs[BK][BN + 1]
// The loaders (supplied by each kernel) fill registers for tile t+1 while the
// matrix cores work on tile t.
// ---------------------------------------------------------------------------
template <int WM_, int WN_, int WK_>
struct TileShape {
  static constexpr int WM = WM_, WN = WN_, WK = WK_;
  static_assert(WM * WN * WK == 4, "4 waves per work-group");
  static constexpr int BM = 32 * WM, BN = 32 * WN, BK = 32 * WK;
  static constexpr int LDA = BM + 1, LDB = BN + 1;
  static constexpr int A_PER_T = BM * BK / kThreads;  // A elements each thread stages
  static constexpr int B_PER_T = BN * BK / kThreads;
  static constexpr int LDS_FLOATS = BK * LDA + BK * LDB;
  static constexpr int RED_FLOATS = (WK - 1) * WM * WN * 64 * 16;
  static_assert(RED_FLOATS <= LDS_FLOATS, "WK reduction reuses the staging area");
};

// One K tile of MFMA work for the calling wave: 16 steps of K = 2.
template <class TS>
__device__ __forceinline__ void mfma_tile(const float* __restrict__ As, const float* __restrict__ Bs,
                                          f32x16& acc, int wm, int wn, int wk, int lane) {
  const int col = lane & 31, khalf = lane >> 5;
  const float* a = As + (wk * 32 + khalf) * TS::LDA + wm * 32 + col;
  const float* b = Bs + (wk * 32 + khalf) * TS::LDB + wn * 32 + col;
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2 * kk * TS::LDA], b[2 * kk * TS::LDB], acc, 0, 0,
                                              0);
  }
}

// Sum the WK partial accumulators of a work-group into the wk == 0 waves.
// Uses `red` (LDS, at least (WK-1) * WM*WN * 64 * 16 floats; the tile staging
// area is large enough) after a barrier.  All threads must call it.
template <class TS>
__device__ __forceinline__ void reduce_wk(f32x16& acc, float* red, int wm, int wn, int wk,
                                          int lane) {
  if constexpr (TS::WK > 1) {
    __syncthreads();
    const int slot = (wm + TS::WM * wn);
    if (wk > 0) {
      float* dst = red + ((wk - 1) * TS::WM * TS::WN + slot) * 64 * 16 + lane;
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[r * 64] = acc[r];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int q = 1; q < TS::WK; ++q) {
        const float* src = red + ((q - 1) * TS::WM * TS::WN + slot) * 64 * 16 + lane;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += src[r * 64];
      }
    }
  }
}

// Row / column of accumulator register r of lane `lane` inside a wave's 32x32 block.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// Kernel launchers (host), one per translation unit's kernels ------------------
ConvGeom make_geom(const cbb_conv_desc& d);
size_t conv_dw_workspace(const ConvGeom& g);
int launch_conv_dw(const ConvGeom& g, const float* x, const float* dz, float* dw, float* ws,
                   hipStream_t st);
int launch_conv_dx(const ConvGeom& g, const float* wt, const float* dz, float* dx, int accumulate,
                   hipStream_t st);
size_t actbn_workspace(int N, int C, int64_t HW);
int launch_actbn(int N, int C, int64_t HW, const float* delta, const float* y, const float* xn,
                 int act, float slope, const float* var, const float* gamma, float eps, int bn,
                 float* dz, float* dgamma, float* dbeta_or_db, void* ws, hipStream_t st);
int launch_act_backward(int act, float slope, const float* y, const float* delta, float* g,
                        int64_t count, hipStream_t st);
int launch_shortcut(int64_t count, float alpha, float beta, const float* delta, float* d_main,
                    float* d_from, hipStream_t st);
int launch_route(int batch, int n_in, const int64_t* sizes, const float* delta,
                 float* const* d_in, hipStream_t st);
int launch_upsample(int n, int c, int h, int w, int scale, const float* delta, float* dx,
                    hipStream_t st);
int launch_maxpool(int n, int c, int ih, int iw, int k, int s, const int32_t* idx,
                   const float* delta, float* dx, hipStream_t st);
int launch_softmax_loss(int batch, int classes, const float* prob, const int32_t* labels,
                        float loss_weight, float* dlogits, int32_t* bad, hipStream_t st);
int launch_fc(int batch, int in_dim, int out_dim, const float* x, const float* w,
              const float* delta, float* dw, float* db, float* dx, int dx_accumulate,
              hipStream_t st);

}  // namespace cbb
