// Weight-only 4-bit projection (paper page, Figures & tables: BF16 and INT4 drafters of equal
// acceptance; explainer, "Where it earns its keep": the drafter's weights quantized to 4 bits).
//
//   out[m][f] = sum_k X[m][k] * (code(f, k) - 8) * scale[f][k / 128]
//
// Codes: two per byte along k (lower k in the low nibble), rows of K/2 bytes; one fp32 scale per
// 128 consecutive k of a row.  A round's projection reads each weight byte once, so the kernel
// streams the packed rows from HBM (a quarter of the bf16 weight bytes) and feeds bf16 MFMAs:
//
// * a workgroup owns 16 output features; its 8 waves split the 128-wide k groups (wave w takes
//   groups w, w + 8, ...), so every group is one 16-row x 64-byte read of the packed weights;
// * inside a group lane l holds 32 codes of row l % 16 (k = 32 (l / 16) .. +31 of the group).
//   The contraction order inside a group is free, so MFMA u (of 4) pairs the lane's k-run
//   32 (l / 16) + 8u .. +7 with the same k-run of the X rows;
// * a code c becomes the bf16 value 128 + c by placing it under the exponent of 128
//   (0x4300 | c), two codes per 32-bit register; one more MFMA per k-run with the constant
//   -136 takes the offset back out, so the group's sum is exact up to fp32 accumulation;
// * the group's sum is scaled by its row's scale and added to the fp32 accumulator; the waves'
//   partial sums meet in LDS at the end and leave as coalesced rows of out.
#include "hyf_launch.h"

namespace hyf {

namespace {

constexpr int W4_GROUP = 128;
constexpr int W4_NW = 8;   // waves per workgroup
constexpr int W4_MROWS = 64;  // X rows one workgroup takes (4 MFMA column tiles)

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Two codes -> two bf16 values 128 + c in one register.
__device__ __forceinline__ uint32_t codes_pair(uint32_t lo, uint32_t hi, int sel) {
  // lo holds codes 0, 2, 4, 6 of a word in its bytes, hi codes 1, 3, 5, 7; sel picks the pair
  // (byte sel of lo -> bits 0..7, byte sel of hi -> bits 16..23)
  const uint32_t pr = __builtin_amdgcn_perm(hi, lo, (0x0cu << 24) | ((4u + sel) << 16) | (0x0cu << 8) | (uint32_t)sel);
  return pr | 0x43004300u;
}

__device__ __forceinline__ bf16x8 codes_frag(uint32_t w) {
  const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
  u32x4 v;
  v[0] = codes_pair(lo, hi, 0);
  v[1] = codes_pair(lo, hi, 1);
  v[2] = codes_pair(lo, hi, 2);
  v[3] = codes_pair(lo, hi, 3);
  return __builtin_bit_cast(bf16x8, v);
}

template <int MT, int FT>
__global__ void __launch_bounds__(W4_NW * 64)
k_linear_w4(RowSrc xs, int M, int K, const uint8_t* __restrict__ Wq, const float* __restrict__ S, int Nout, Epi epi) {
  __shared__ float red[W4_NW * FT * MT * 256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (epi.zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int z = threadIdx.x; z < epi.n_zero; z += W4_NW * 64) epi.zero[z] = 0;
  const int i = lane & 15, g = lane >> 4;
  const int f0 = blockIdx.x * 16 * FT;  // FT tiles of 16 features, sharing the X fragments
  const int m0 = blockIdx.y * W4_MROWS;
  const int ng = K / W4_GROUP;
  // rows past Nout read the last row (their results are never stored)
  const uint8_t* wrow[FT];
  const float* srow[FT][4];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    wrow[ft] = Wq + (int64_t)min(f0 + 16 * ft + i, Nout - 1) * (K / 2) + 16 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) srow[ft][r] = S + (int64_t)min(f0 + 16 * ft + 4 * g + r, Nout - 1) * ng;
  }
  const bf16* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m0 + 16 * t + i;
    xok[t] = m < M;
    xrow[t] = static_cast<const bf16*>(row_ptr(xs, xok[t] ? m : 0, K, 2)) + 32 * g;
  }
  const bf16x8 neg136 = __builtin_bit_cast(bf16x8, u32x4{0xc308c308u, 0xc308c308u, 0xc308c308u, 0xc308c308u});
  f32x4 acc[FT][MT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[ft][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A wave takes its groups DEPTH at a time: every load of the DEPTH groups (codes, scales, X
  // fragments) is issued before the first MFMA, so the wave waits one memory latency per DEPTH
  // groups rather than one per group.
  constexpr int DEPTH = MT >= 4 ? 1 : 4 / MT;
  for (int base = wave; base < ng; base += W4_NW * DEPTH) {
    u32x4 w[FT][DEPTH];
    float sc[FT][DEPTH][4];
    bf16x8 xb[DEPTH][MT][4];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int grp = base + d * W4_NW;
      const bool ok = grp < ng;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        w[ft][d] = ok ? *reinterpret_cast<const u32x4*>(wrow[ft] + (int64_t)grp * 64) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[ft][d][r] = ok ? srow[ft][r][grp] : 0.f;
      }
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          xb[d][t][u] = ok && xok[t] ? *reinterpret_cast<const bf16x8*>(xrow[t] + grp * W4_GROUP + 8 * u) : bf16x8{};
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (base + d * W4_NW >= ng) break;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        bf16x8 a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = codes_frag(w[ft][d][u]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], xb[d][t][u], part, 0, 0, 0);
            part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(neg136, xb[d][t][u], part, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ft][t][r] += part[r] * sc[ft][d][r];
        }
      }
    }
  }
  // partial sums of the waves: element (r, lane) of tile (ft, t) is feature
  // f0 + 16 ft + 4 (lane / 16) + r, row m0 + 16 t + lane % 16
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(((wave * FT + ft) * MT + t) * 4 + r) * 64 + lane] = acc[ft][t][r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < FT * MT * 256; idx += W4_NW * 64) {
    const int t = idx >> 8, e = idx & 255;  // e: 16 features (fastest) x 16 rows of one m tile
    const int fl = e & 15, ml = e >> 4;
    const int src_lane = (fl >> 2) * 16 + ml, r = fl & 3;
    const int ft = t / MT, tm = t % MT;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < W4_NW; ++w) v += red[(((w * FT + ft) * MT + tm) * 4 + r) * 64 + src_lane];
    const int f = f0 + 16 * ft + fl, m = m0 + 16 * tm + ml;
    if (f < Nout && m < M) epi_store<bf16>(epi, m, f, v);
  }
}

template <int FT>
void launch_w4_mt(int mt, dim3 grid, const RowSrc& x, int64_t M, int K, const uint8_t* Wq, const float* S, int Nout,
                  const Epi& epi, hipStream_t s) {
  const dim3 block(W4_NW * 64);
  switch (mt) {
    case 1: hipLaunchKernelGGL((k_linear_w4<1, FT>), grid, block, 0, s, x, (int)M, K, Wq, S, Nout, epi); break;
    case 2: hipLaunchKernelGGL((k_linear_w4<2, FT>), grid, block, 0, s, x, (int)M, K, Wq, S, Nout, epi); break;
    case 3: hipLaunchKernelGGL((k_linear_w4<3, FT>), grid, block, 0, s, x, (int)M, K, Wq, S, Nout, epi); break;
    default: hipLaunchKernelGGL((k_linear_w4<4, FT>), grid, block, 0, s, x, (int)M, K, Wq, S, Nout, epi); break;
  }
}

// out[f][k] = bf16((code(f, k) - 8) * scale[f][k / 128]): one byte (two codes) per thread.
__global__ void __launch_bounds__(256) k_w4_dequant(const uint8_t* __restrict__ Wq, const float* __restrict__ S,
                                                    int64_t bytes, int K, bf16* __restrict__ out) {
  const int half = K / 2, ng = K / W4_GROUP;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < bytes; i += (int64_t)gridDim.x * 256) {
    const int64_t f = i / half;
    const int j = (int)(i % half);
    const uint32_t b = Wq[i];
    const float sc = S[f * ng + (2 * j) / W4_GROUP];
    out[f * K + 2 * j] = static_cast<bf16>((float)((int)(b & 15u) - 8) * sc);
    out[f * K + 2 * j + 1] = static_cast<bf16>((float)((int)(b >> 4) - 8) * sc);
  }
}

}  // namespace

hipError_t launch_linear_w4_epi(const RowSrc& x, int64_t M, int K, const uint8_t* Wq, const float* S, int Nout,
                                const Epi& epi, hipStream_t s) {
  if (M <= 0 || Nout <= 0) return hipSuccess;
  if (epi.trans) return hipErrorInvalidValue;  // the time-blocked layout is the prefill GEMM's
  const int mt = (int)((M < W4_MROWS ? M : W4_MROWS) + 15) / 16;
  const int tiles = (Nout + 15) / 16;
  const unsigned gy = (unsigned)((M + W4_MROWS - 1) / W4_MROWS);
  // One workgroup fits a CU at this kernel's register count: past one workgroup per CU, two
  // feature tiles per workgroup keep the grid to one round (and share the X fragments).
  if (tiles > 256 && mt <= 2)
    launch_w4_mt<2>(mt, dim3((tiles + 1) / 2, gy), x, M, K, Wq, S, Nout, epi, s);
  else
    launch_w4_mt<1>(mt, dim3(tiles, gy), x, M, K, Wq, S, Nout, epi, s);
  return hipGetLastError();
}

hipError_t launch_linear_w4(const bf16* X, int64_t M, int K, const uint8_t* Wq, const float* S, int Nout,
                            void* out, bool out_f32, hipStream_t s) {
  RowSrc xs{X, X, M};
  Epi e{out, Nout, out_f32 ? 1 : 0, Nout, nullptr, 0, 0, nullptr, 0};
  return launch_linear_w4_epi(xs, M, K, Wq, S, Nout, e, s);
}

hipError_t launch_w4_dequant(const uint8_t* Wq, const float* S, int rows, int K, bf16* out, hipStream_t s) {
  const int64_t bytes = (int64_t)rows * (K / 2);
  if (bytes <= 0) return hipSuccess;
  const int64_t want = (bytes + 255) / 256;
  hipLaunchKernelGGL(k_w4_dequant, dim3((unsigned)(want < 4096 ? want : 4096)), dim3(256), 0, s, Wq, S, bytes, K, out);
  return hipGetLastError();
}

}  // namespace hyf
