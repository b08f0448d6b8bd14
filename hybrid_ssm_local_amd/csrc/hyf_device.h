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
// rows row0[i] .. row0[i+1] of the call's commit-row space; in time-blocked buffers its tokens
// start at block blk0[i] (blocks of HYF_TBLK tokens); seg0 indexes scan segments.
struct ReqTable {
  int32_t n_req;
  int32_t slot[HYF_MAX_REQUESTS];
  int32_t row0[HYF_MAX_REQUESTS + 1];
  int32_t blk0[HYF_MAX_REQUESTS + 1];
  int32_t seg0[HYF_MAX_REQUESTS + 1];
};

// Tiled time-blocked layout of the scan's MFMA operands x and B.  A block holds HYF_TBLK tokens of
// F features (F a multiple of 16).  Features come in groups of 16 and tokens in runs of
// KT = 4 VN, where VN = 16 / sizeof(T) tokens fill 16 bytes; a 16 x KT tile is 4 slices of VN
// tokens, and slice s holds, feature by feature, VN consecutive tokens.  One tile is thus the
// 16-byte chunks that the 64 lanes of one 16x16 MFMA load, in lane order (1 KiB, contiguous).
// Returns the element offset of (feature f, token t < HYF_TBLK) inside its block.
template <typename T>
__host__ __device__ __forceinline__ int64_t tile_off(int64_t f, int t) {
  constexpr int VN = 16 / (int)sizeof(T), KT = 4 * VN, NJ = HYF_TBLK / KT;
  return (((f / 16) * NJ + t / KT) * 64 + ((t % KT) / VN) * 16 + f % 16) * VN + t % VN;
}

// Static layer shape as the kernels see it.
struct Shape {
  int32_t d, nh, P, N, G, W, L, cross;
  int32_t dq, gn, n_in;
  int32_t gdn;  // 1: gated delta-rule memory (gates alpha at off_dt, beta at off_beta), 0: Mamba-2
  int32_t w4;   // 1: the projections' weights are 4-bit codes and scales
  int32_t lastw;  // 1: Mamba-2 over the last W committed rows (B and step rings in the state)
  // w_in row offsets of each group
  int32_t off_q, off_c, off_k, off_v, off_b, off_dt, off_beta;
  // state blob
  uint64_t st_bytes, st_h, st_k, st_v, st_b, st_dt;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

__device__ __forceinline__ float softplus_f(float z) {
  // log(1 + e^z) without overflow: max(z, 0) + log(1 + e^-|z|), on the hardware exp2/log2 (their
  // error, a few 1e-7 relative, is far inside every tolerance the results are held to; where
  // e^-|z| drops below fp32's epsilon the result is max(z, 0) to within that epsilon)
  return fmaxf(z, 0.f) + __logf(1.f + __expf(-fabsf(z)));
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

// The same reductions without LDS traffic: DPP moves inside each 16-lane row (swaps inside quads,
// the mirrored half-row, the mirrored row), then the four row results read as scalars.  The result
// is uniform (every lane gets it).
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
__device__ __forceinline__ float wave_sum64(float v) {
  v += dpp_row<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_row<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_row<0x141>(v);  // row_half_mirror
  v += dpp_row<0x140>(v);  // row_mirror
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
__device__ __forceinline__ float wave_max64(float v) {
  v = fmaxf(v, dpp_row<0xB1>(v));
  v = fmaxf(v, dpp_row<0x4E>(v));
  v = fmaxf(v, dpp_row<0x141>(v));
  v = fmaxf(v, dpp_row<0x140>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
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

// Wait until at most N vector-memory operations of this wave are outstanding (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until this wave's LDS (and scalar-memory) operations are done: lgkmcnt(0), vmcnt and
// expcnt at their no-wait maxima.
__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Direct global -> LDS loads (no registers): lane l's 16 (or 4) bytes land at lds_base + 16 l
// (4 l).  lds_base must be the same for the whole wave; the data is there once this wave's
// vector-memory count drains (vm_wait<0>) — other waves see it after a barrier.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src),
                                   (void __attribute__((address_space(3)))*)(lds_base), 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src),
                                   (void __attribute__((address_space(3)))*)(lds_base), 4, 0, 0);
}

// A staging job of n 16-byte chunks, chunk i from global src(i) to LDS dst + 16 i, by a workgroup
// of THREADS threads with direct global -> LDS loads: no registers and no wait between loads, so
// all jobs a workgroup issues before its vm_wait<0>() + barrier cost one memory round trip.  A
// wave issues chunks [64 k, 64 k + 64) for k = wave, wave + THREADS / 64, ...; lanes past n are
// masked off.  aux: cache policy bits of the loads.
template <int THREADS, int AUX = 0, typename F>
__device__ __forceinline__ void lds_stage16(int n, void* dst, F src) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int base = wave * 64; base < n; base += THREADS)
    if (base + lane < n)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src(base + lane)),
                                       (void __attribute__((address_space(3)))*)(static_cast<char*>(dst) + 16 * base),
                                       16, 0, AUX);
}

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
