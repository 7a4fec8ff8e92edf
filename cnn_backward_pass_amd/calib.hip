// calib.hip -- libcbb_calib.so: the two on-box peak probes the benchmark reports
// fractions against (measurement only; no part of the backward pass).
//
//   calib_mfma_f32  every wave issues `iters` rounds of four independent
//                   v_mfma_f32_32x32x2_f32 chains from registers (no memory
//                   traffic in the loop): the fp32 matrix rate the chip sustains
//                   at the clock it holds under that load.
//   calib_copy      a 16-byte-per-lane grid-stride device copy (non-temporal
//                   loads and stores, 1-4 pieces per lane in flight): the HBM
//                   rate of one read and one write stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void calib_mfma_kernel(int iters, float* __restrict__ out) {
  const float a = (float)(threadIdx.x + 1) * 1e-3f, b = (float)(blockIdx.x + 1) * 1e-3f;
  f32x16 c0, c1, c2, c3;
#pragma unroll
  for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// U 16-byte pieces per lane in flight per iteration (all loads issued before the stores).
template <int U>
__global__ __launch_bounds__(256) void calib_copy_kernel(const f4* __restrict__ src,
                                                         f4* __restrict__ dst, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n4; i += U * stride) {
    f4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n4; i += stride) dst[i] = src[i];
}

extern "C" {

// FLOPs of one call: blocks * 4 waves * iters * 4 chains * (32*32*2*2).
// out: blocks * 256 floats of device memory.  0, or -1 on bad arguments / launch error.
int calib_mfma_f32(int blocks, int iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out) return -1;
  calib_mfma_kernel<<<blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Copies `bytes` (a multiple of 16, both pointers 16-byte aligned, no overlap) with
// `blocks` work-groups (<= 0: one pass of 256 lanes x 16 bytes each) and `unroll`
// pieces per lane in flight (1, 2 or 4).
int calib_copy(const void* src, void* dst, int64_t bytes, int blocks, int unroll, void* stream) {
  if (!src || !dst || bytes < 16 || bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) % 16)
    return -1;
  const int64_t n4 = bytes / 16;
  int64_t nb = blocks > 0 ? blocks : (n4 + 255) / 256;
  if (nb > (1 << 20)) nb = 1 << 20;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const f4* s4 = static_cast<const f4*>(src);
  f4* d4 = static_cast<f4*>(dst);
  switch (unroll) {
    case 1: calib_copy_kernel<1><<<(unsigned)nb, 256, 0, st>>>(s4, d4, n4); break;
    case 2: calib_copy_kernel<2><<<(unsigned)nb, 256, 0, st>>>(s4, d4, n4); break;
    case 4: calib_copy_kernel<4><<<(unsigned)nb, 256, 0, st>>>(s4, d4, n4); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
