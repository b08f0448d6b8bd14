// Device-side helpers shared by the libhyflash kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hyflash.h"

namespace hyf {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// Per-call request table, passed by value in the kernel arguments (no host->device copy, so
// a call can be captured in a graph).  Request i owns pool blob slot[i]; its commit rows are
// rows row0[i] .. row0[i+1] of the call's commit-row space; seg0 indexes scan segments.
struct ReqTable {
  int32_t n_req;
  int32_t slot[HYF_MAX_REQUESTS];
  int32_t row0[HYF_MAX_REQUESTS + 1];
  int32_t seg0[HYF_MAX_REQUESTS + 1];
};

// Static layer shape as the kernels see it.
struct Shape {
  int32_t d, nh, P, N, G, W, L, cross;
  int32_t dq, gn, n_in;
  // w_in row offsets of each group
  int32_t off_q, off_c, off_k, off_v, off_b, off_dt;
  // state blob
  uint64_t st_bytes, st_h, st_k, st_v;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

__device__ __forceinline__ float softplus_f(float z) {
  // log(1 + e^z) without overflow: max(z, 0) + log1p(exp(-|z|)).
  return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}

// 64-lane wave reductions (all lanes get the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------------------------
// MFMA 16x16 tiles.  Layouts (checked on gfx950):
//   bf16 16x16x32: lane l supplies A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16];
//   f32  16x16x4 : lane l supplies A[l%16][l/16] and B[l/16][l%16];
//   both: lane l receives C[4*(l/16) + r][l%16], r = 0..3.
// The reduction index k only has to be permuted the same way on both operands, so a lane
// may take its k values from any fixed positions; the kernels give each lane a contiguous run.
template <typename T> struct Mfma16;

template <> struct Mfma16<bf16> {
  static constexpr int KE = 8;  // k values one lane supplies per instruction
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma16<float> {
  static constexpr int KE = 1;
  typedef float frag;
  __device__ __forceinline__ static f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// 16-byte vector of storage elements.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> {
  static constexpr int n = 8;
  typedef bf16x8 type;
};
template <> struct Vec16<float> {
  static constexpr int n = 4;
  typedef f32x4 type;
};

}  // namespace hyf
