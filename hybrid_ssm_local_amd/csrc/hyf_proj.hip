// Projections of the drafter layer: out[m][f] = sum_k X[m][k] * W[f][k].
//
// Kernels, chosen by the number of rows M:
//  * k_proj_stream (bf16) and k_proj_small (fp32), M <= 64: the batch-1 round.  The layer's
//    weights are read from HBM exactly once; every 16 output features are one workgroup whose
//    waves split K into slabs and reduce their partial tiles through LDS in a fixed order
//    (deterministic).  MFMA 16x16 tiles: W is the A operand (16 features), X^T the B operand
//    (16 rows per tile).
//  * k_gemm_bf16_256 (large M, K a multiple of 64; hyf_gemm.hip): prefill and batched rounds.
//    256x128 macro tiles, three LDS stages filled by direct global -> LDS copies, 8 waves of 64x64
//    each built from 16x16x32 bf16 MFMAs.
//  * k_gemm_bf16 (large M, other K): 128x128 macro tiles, K step 64, register-staged
//    double-buffered LDS, 4 waves of 64x64.
#include <mutex>

#include "hyf_launch.h"

namespace hyf {

template <typename T>
__device__ __forceinline__ typename Vec16<T>::type ld_vec(const T* p) {
  return *reinterpret_cast<const typename Vec16<T>::type*>(p);
}

// ---------------------------------------------------------------------------------------------
template <typename T, int NW, int MT>
__global__ void __launch_bounds__(NW * 64)
k_proj_small(RowSrc xs, int M, int K, const T* __restrict__ W, int Nout, Epi epi) {
  constexpr int KE = Mfma16<T>::KE;
  constexpr int VN = Vec16<T>::n;
  constexpr int U = 4;                // MFMAs per slab
  constexpr int LANE_K = U * KE;      // k values a lane covers per slab
  constexpr int NV = LANE_K / VN;     // 16-byte loads per lane per slab and operand row
  constexpr int SLAB = 4 * LANE_K;    // k per slab
  typedef typename Vec16<T>::type V;
  typedef typename Mfma16<T>::frag Fr;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int f0 = blockIdx.x * 16;
  if (epi.zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int z = threadIdx.x; z < epi.n_zero; z += NW * 64) epi.zero[z] = 0;
  const int m_base = blockIdx.y * 16 * MT;

  const T* wrow = W + (int64_t)min(f0 + i, Nout - 1) * K;
  const T* xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(m_base + mt * 16 + i, M - 1);
    xrow[mt] = static_cast<const T*>(row_ptr(xs, m, K, sizeof(T)));
  }

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A wave takes slabs wave, wave + NW, ...; it loads SB of them before it multiplies, so a whole
  // row of weights is in flight at once (same order of MFMAs as one slab at a time).
  constexpr int SB = MT == 1 ? 3 : 1;  // at most 128 VGPRs: two 8-wave workgroups per CU
  const int nslab = (K + SLAB - 1) / SLAB;
  for (int s0 = wave; s0 < nslab; s0 += SB * NW) {
    V wv[SB][NV];
    V xv[SB][MT][NV];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      // load v of lane group g: k = slab start + 4 VN v + VN g, so the four groups read 64
      // contiguous bytes of every row (MFMA u contracts the 4 VN k values of load u)
      const int kb = (s0 + sb * NW) * SLAB + g * VN;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int k = kb + v * 4 * VN;
        const bool ok = k + VN <= K;
        wv[sb][v] = ok ? ld_vec<T>(wrow + k) : V{};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) xv[sb][mt][v] = ok ? ld_vec<T>(xrow[mt] + k) : V{};
      }
    }
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        Fr a;
        if constexpr (KE == 8) a = wv[sb][u]; else a = wv[sb][0][u];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          Fr b;
          if constexpr (KE == 8) b = xv[sb][mt][u]; else b = xv[sb][mt][0][u];
          acc[mt] = Mfma16<T>::mma(a, b, acc[mt]);
        }
      }
    }
  }

  // Cross-wave reduction in a fixed order.
  __shared__ float red[NW][MT][4][64];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][mt][r][lane] = acc[mt][r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < MT * 256; idx += NW * 64) {
    const int mt = idx >> 8, rem = idx & 255;
    const int fl = rem & 15, ml = rem >> 4;
    const int src_lane = (fl >> 2) * 16 + ml, r = fl & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[w][mt][r][src_lane];
    const int f = f0 + fl;
    const int m = m_base + mt * 16 + ml;
    if (f < Nout && m < M) epi_store<T>(epi, m, f, v);
  }
}

// ---------------------------------------------------------------------------------------------
// bf16, M <= 64: the same K split and MFMA order as k_proj_small (bit-identical results), but the
// weight rows and the x rows of a slab reach LDS by direct loads: one instruction moves 4 rows x
// 256 contiguous bytes (the register path moves 16 rows x 64 bytes per instruction, which costs
// the address unit twice as many cycles per byte).  Slot (r, p) of a 16-row x 256-byte tile holds
// the row's 16-byte chunk p ^ r, so the fragment reads of 16 lanes (16 rows, one chunk) fall in 16
// different bank groups.  Each wave owns its LDS region, so only its own load count is waited on.
constexpr int PS_SLAB = 128;  // k per slab: 256 bytes of a row

template <int NW, int MT>
__global__ void __launch_bounds__(NW * 64)
k_proj_stream(RowSrc xs, int M, int K, const bf16* __restrict__ W, int Nout, Epi epi) {
  constexpr int XT = MT < 2 ? MT : 2;  // x tiles staged at once
  constexpr int PASSES = (MT + XT - 1) / XT;
  constexpr int PER = 4096 * (1 + XT);  // LDS bytes per wave: the weight tile and XT x tiles
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int p = lane & 15, r4 = lane >> 4;  // the lane's slot in a direct-load instruction
  const int f0 = blockIdx.x * 16;
  if (epi.zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int z = threadIdx.x; z < epi.n_zero; z += NW * 64) epi.zero[z] = 0;
  const int m_base = blockIdx.y * 16 * MT;
  char* wl = smem + wave * PER;
  char* xl = wl + 4096;

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nslab = (K + PS_SLAB - 1) / PS_SLAB;
  for (int s = wave; s < nslab; s += NW) {
    const int kb = s * PS_SLAB;
    lgkm_wait0();  // the previous slab's fragment reads are done before its regions are refilled
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * j + r4;
      const int k = kb + ((p ^ r) << 3);
      if (k < K) lds_dma16(W + (int64_t)min(f0 + r, Nout - 1) * K + k, wl + j * 1024);
    }
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      if (ps > 0) lgkm_wait0();
#pragma unroll
      for (int xt = 0; xt < XT; ++xt) {
        const int mt = ps * XT + xt;
        if (mt < MT) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = 4 * j + r4;
            const int m = m_base + mt * 16 + r;
            const int k = kb + ((p ^ r) << 3);
            // rows past M stay unloaded: they only feed output columns that are never stored
            if (m < M && k < K)
              lds_dma16(static_cast<const bf16*>(row_ptr(xs, m, K, 2)) + k, xl + xt * 4096 + j * 1024);
          }
        }
      }
      vm_wait<0>();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // MFMA u contracts k = kb + 32 u + 8 g .. + 7 (chunk g + 4 u), as k_proj_small does; chunks
        // past K are zero on both operands
        const int c = g + 4 * u;
        const bool ok = kb + c * 8 < K;
        const int o = i * 256 + ((c ^ i) << 4);
        const bf16x8 a = ok ? *reinterpret_cast<const bf16x8*>(wl + o) : bf16x8{};
#pragma unroll
        for (int xt = 0; xt < XT; ++xt) {
          const int mt = ps * XT + xt;
          if (mt < MT) {
            const bf16x8 b = ok ? *reinterpret_cast<const bf16x8*>(xl + xt * 4096 + o) : bf16x8{};
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[mt], 0, 0, 0);
          }
        }
      }
    }
  }

  // Cross-wave reduction in a fixed order (the LDS regions are free once every wave is here).
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [NW][MT][4][64]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((wave * MT + mt) * 4 + r) * 64 + lane] = acc[mt][r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < MT * 256; idx += NW * 64) {
    const int mt = idx >> 8, rem = idx & 255;
    const int fl = rem & 15, ml = rem >> 4;
    const int src_lane = (fl >> 2) * 16 + ml, r = fl & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[((w * MT + mt) * 4 + r) * 64 + src_lane];
    const int f = f0 + fl;
    const int m = m_base + mt * 16 + ml;
    if (f < Nout && m < M) epi_store<bf16>(epi, m, f, v);
  }
}

// One 16-row tile of X with a grid of at most one workgroup per CU (w_out of a round): the same
// slabs, waves and MFMA order as k_proj_stream<NW, 1> (so the same bits), with two LDS buffers per
// wave: the next slab's direct loads are in flight while the current slab's MFMAs run.  Every slab
// issues exactly 8 loads (addresses past M or K are clamped to valid ones; such chunks feed only
// zeroed fragments or output columns that are never stored), so waiting until at most 8 loads
// are outstanding means the current slab has landed.
template <int NW>
__global__ void __launch_bounds__(NW * 64)
k_proj_stream2(RowSrc xs, int M, int K, const bf16* __restrict__ W, int Nout, Epi epi) {
  constexpr int PER = 8192;  // LDS bytes per wave and buffer: the weight tile and one x tile
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int p = lane & 15, r4 = lane >> 4;
  const int f0 = blockIdx.x * 16;
  if (epi.zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int z = threadIdx.x; z < epi.n_zero; z += NW * 64) epi.zero[z] = 0;
  const int m_base = blockIdx.y * 16;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nslab = (K + PS_SLAB - 1) / PS_SLAB;
  auto issue = [&](int sl, int buf) {
    char* wl = smem + (wave * 2 + buf) * PER;
    char* xl = wl + 4096;
    const int kb = sl * PS_SLAB;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * j + r4;
      const int k = min(kb + ((p ^ r) << 3), K - 8);
      lds_dma16(W + (int64_t)min(f0 + r, Nout - 1) * K + k, wl + j * 1024);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * j + r4;
      const int m = min(m_base + r, M - 1);
      const int k = min(kb + ((p ^ r) << 3), K - 8);
      lds_dma16(static_cast<const bf16*>(row_ptr(xs, m, K, 2)) + k, xl + j * 1024);
    }
  };
  if (wave < nslab) issue(wave, 0);
  int it = 0;
  for (int sl = wave; sl < nslab; sl += NW, ++it) {
    if (sl + NW < nslab) {
      lgkm_wait0();  // the fragment reads of the buffer about to be refilled are done
      issue(sl + NW, (it + 1) & 1);
      vm_wait<8>();
    } else {
      vm_wait<0>();
    }
    const char* wl = smem + (wave * 2 + (it & 1)) * PER;
    const char* xl = wl + 4096;
    const int kb = sl * PS_SLAB;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = g + 4 * u;
      const bool ok = kb + c * 8 < K;
      const int o = i * 256 + ((c ^ i) << 4);
      const bf16x8 a = ok ? *reinterpret_cast<const bf16x8*>(wl + o) : bf16x8{};
      const bf16x8 b = ok ? *reinterpret_cast<const bf16x8*>(xl + o) : bf16x8{};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
  }
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [NW][4][64]
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 256; idx += NW * 64) {
    const int fl = idx & 15, ml = idx >> 4;
    const int src_lane = (fl >> 2) * 16 + ml, r = fl & 3;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[(w * 4 + r) * 64 + src_lane];
    const int f = f0 + fl;
    const int m = m_base + ml;
    if (f < Nout && m < M) epi_store<bf16>(epi, m, f, v);
  }
}

// ---------------------------------------------------------------------------------------------
// bf16 GEMM, 128x128 macro tile, K step 64.
constexpr int GB_M = 128, GB_N = 128, GB_K = 64, GB_LD = GB_K + 8;  // LDS row pitch (elements)

__device__ __forceinline__ void gemm_load_tile(const RowSrc& xs, int M, int K, const bf16* W, int Nout,
                                               int m0, int n0, int k0, bf16x8 (&ra)[4], bf16x8 (&rb)[4]) {
  const int t = threadIdx.x;
  const int gcol = (t & 7) * 8;
  const int k = k0 + gcol;
  const bool kok = k + 8 <= K;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (t >> 3) + 32 * j;
    const int m = min(m0 + row, M - 1);
    const bf16* xr = static_cast<const bf16*>(row_ptr(xs, m, K, 2));
    ra[j] = kok ? *reinterpret_cast<const bf16x8*>(xr + k) : bf16x8{};
    const int f = min(n0 + row, Nout - 1);
    rb[j] = kok ? *reinterpret_cast<const bf16x8*>(W + (int64_t)f * K + k) : bf16x8{};
  }
}

__device__ __forceinline__ void gemm_store_lds(bf16* la, bf16* lb, const bf16x8 (&ra)[4], const bf16x8 (&rb)[4]) {
  const int t = threadIdx.x;
  const int gcol = (t & 7) * 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (t >> 3) + 32 * j;
    *reinterpret_cast<bf16x8*>(la + row * GB_LD + gcol) = ra[j];
    *reinterpret_cast<bf16x8*>(lb + row * GB_LD + gcol) = rb[j];
  }
}

template <typename TO>
__global__ void __launch_bounds__(256)
k_gemm_bf16(RowSrc xs, int M, int K, const bf16* __restrict__ W, int Nout, Epi epi) {
  __shared__ __attribute__((aligned(16))) bf16 lds[2][2][GB_M * GB_LD];  // [buf][A/B]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * GB_N, m0 = blockIdx.y * GB_M;
  if (epi.zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int z = threadIdx.x; z < epi.n_zero; z += 256) epi.zero[z] = 0;

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 ra[4], rb[4];
  const int nk = (K + GB_K - 1) / GB_K;
  gemm_load_tile(xs, M, K, W, Nout, m0, n0, 0, ra, rb);
  gemm_store_lds(lds[0][0], lds[0][1], ra, rb);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gemm_load_tile(xs, M, K, W, Nout, m0, n0, (kt + 1) * GB_K, ra, rb);
    const bf16* la = lds[cur][0];
    const bf16* lb = lds[cur][1];
#pragma unroll
    for (int ks = 0; ks < GB_K / 32; ++ks) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        fa[t] = *reinterpret_cast<const bf16x8*>(la + (wm * 64 + t * 16 + i) * GB_LD + ks * 32 + g * 8);
        fb[t] = *reinterpret_cast<const bf16x8*>(lb + (wn * 64 + t * 16 + i) * GB_LD + ks * 32 + g * 8);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < nk) gemm_store_lds(lds[cur ^ 1][0], lds[cur ^ 1][1], ra, rb);
    __syncthreads();
  }
  if (epi.trans) {
    // Time-blocked output: the 128-row tile is one block (m0 is a multiple of 128).  Stage the fp32
    // tile as [f][m] in LDS, then write 8 tokens of one feature per item: one 16-byte chunk of the
    // tiled layout for out0 (consecutive items take consecutive features, so 16 of them fill a
    // contiguous 256 bytes), two 16-byte runs of the plain [f][HYF_TBLK] rows for out1.
    constexpr int CP = GB_M + 4;  // float pitch
    float* ct = reinterpret_cast<float*>(&lds[0][0][0]);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ct[(wn * 64 + b * 16 + i) * CP + wm * 64 + a * 16 + 4 * g + r] = acc[a][b][r];
    __syncthreads();
    for (int it = threadIdx.x; it < GB_N * (GB_M / 8); it += 256) {
      const int fl = it % GB_N, m8 = (it / GB_N) * 8;
      const int f = n0 + fl;
      const int64_t m = (int64_t)m0 + m8;
      if (f >= Nout || m >= M) continue;
      const float* src = ct + fl * CP + m8;
      if (m + 8 <= M) {
        const int64_t blk = m0 / GB_M;
        if (f < epi.n_split && !epi.out0_f32) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = static_cast<bf16>(src[e]);
          *reinterpret_cast<bf16x8*>(static_cast<bf16*>(epi.out0) + blk * epi.ld0 + tile_off<bf16>(f, m8)) = v;
        } else {
          float* dst = f < epi.n_split ? static_cast<float*>(epi.out0) + blk * epi.ld0 + (int64_t)f * GB_M + m8
                                       : epi.out1 + blk * epi.ld1 + (int64_t)(f - epi.n_split) * GB_M + m8;
          *reinterpret_cast<f32x4*>(dst) = f32x4{src[0], src[1], src[2], src[3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{src[4], src[5], src[6], src[7]};
        }
      } else {
        for (int e = 0; m + e < M; ++e) epi_store<TO>(epi, m + e, f, src[e]);
      }
    }
    return;
  }
  // lane holds C[4g + r][i] of tile (a, b): row m, column f.
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + a * 16 + 4 * g + r;
        const int f = n0 + wn * 64 + b * 16 + i;
        if (m < M && f < Nout) epi_store<TO>(epi, m, f, acc[a][b][r]);
      }
}

// ---------------------------------------------------------------------------------------------
template <typename T, int NW>
static hipError_t launch_small_nw(RowSrc x, int M, int K, const T* W, int Nout, const Epi& epi, hipStream_t s) {
  const int mt = (M + 15) / 16;
  const int MT = mt >= 4 ? 4 : mt;
  dim3 grid((Nout + 15) / 16, (M + 16 * MT - 1) / (16 * MT));
  dim3 block(NW * 64);
  switch (MT) {
    case 1: hipLaunchKernelGGL((k_proj_small<T, NW, 1>), grid, block, 0, s, x, M, K, W, Nout, epi); break;
    case 2: hipLaunchKernelGGL((k_proj_small<T, NW, 2>), grid, block, 0, s, x, M, K, W, Nout, epi); break;
    case 3: hipLaunchKernelGGL((k_proj_small<T, NW, 3>), grid, block, 0, s, x, M, K, W, Nout, epi); break;
    default: hipLaunchKernelGGL((k_proj_small<T, NW, 4>), grid, block, 0, s, x, M, K, W, Nout, epi); break;
  }
  return hipGetLastError();
}

template <int NW, int MT>
static hipError_t launch_stream_t(RowSrc x, int M, int K, const bf16* W, int Nout, const Epi& epi, hipStream_t s) {
  constexpr int XT = MT < 2 ? MT : 2;
  const size_t lds = (size_t)NW * 4096 * (1 + XT);
  static std::once_flag once;
  static hipError_t set_err = hipSuccess;
  std::call_once(once, [] {
    set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_proj_stream<NW, MT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
  });
  if (set_err != hipSuccess) return set_err;
  dim3 grid((Nout + 15) / 16, (M + 16 * MT - 1) / (16 * MT));
  hipLaunchKernelGGL((k_proj_stream<NW, MT>), grid, dim3(NW * 64), lds, s, x, M, K, W, Nout, epi);
  return hipGetLastError();
}

template <int NW>
static hipError_t launch_stream2(RowSrc x, int M, int K, const bf16* W, int Nout, const Epi& epi, hipStream_t s) {
  const size_t lds = (size_t)NW * 2 * 8192;
  static std::once_flag once;
  static hipError_t set_err = hipSuccess;
  std::call_once(once, [] {
    set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_proj_stream2<NW>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
  });
  if (set_err != hipSuccess) return set_err;
  hipLaunchKernelGGL((k_proj_stream2<NW>), dim3((Nout + 15) / 16, 1), dim3(NW * 64), lds, s, x, M, K, W, Nout, epi);
  return hipGetLastError();
}

template <int NW>
static hipError_t launch_stream_nw(RowSrc x, int M, int K, const bf16* W, int Nout, const Epi& epi, hipStream_t s) {
  const int mt = (M + 15) / 16;
  // One row tile on at most 256 workgroups (one per CU): the double-buffered kernel (the same
  // results); larger grids keep more workgroups per CU in flight with the single buffer instead.
  if (NW == 8 && mt == 1 && Nout <= 4096) return launch_stream2<NW>(x, M, K, W, Nout, epi, s);
  switch (mt >= 4 ? 4 : mt) {
    case 1: return launch_stream_t<NW, 1>(x, M, K, W, Nout, epi, s);
    case 2: return launch_stream_t<NW, 2>(x, M, K, W, Nout, epi, s);
    case 3: return launch_stream_t<NW, 3>(x, M, K, W, Nout, epi, s);
    default: return launch_stream_t<NW, 4>(x, M, K, W, Nout, epi, s);
  }
}

template <typename T>
static hipError_t launch_small(RowSrc x, int M, int K, const T* W, int Nout, const Epi& epi, hipStream_t s) {
  // The split of K over waves depends on K alone, so an output element is reduced in the same
  // order whatever rows and columns share the launch (a fused round and a standalone commit give
  // bit-identical projections).  Long rows use 8 waves to keep more loads in flight.
  if constexpr (sizeof(T) == 2) {
    if (K >= 2048) return launch_stream_nw<8>(x, M, K, W, Nout, epi, s);
    return launch_stream_nw<4>(x, M, K, W, Nout, epi, s);
  } else {
    if (K >= 2048) return launch_small_nw<T, 8>(x, M, K, W, Nout, epi, s);
    return launch_small_nw<T, 4>(x, M, K, W, Nout, epi, s);
  }
}

hipError_t launch_linear(int dtype, RowSrc x, int64_t M, int K, const void* W, int Nout, const Epi& epi,
                         hipStream_t s) {
  if (M <= 0 || Nout <= 0) return hipSuccess;
  if (dtype == HYF_BF16) {
    if (M <= 64 && !epi.trans) return launch_small<bf16>(x, (int)M, K, static_cast<const bf16*>(W), Nout, epi, s);
    if (K % 64 == 0) return launch_gemm256(x, (int)M, K, static_cast<const bf16*>(W), Nout, epi, s);
    dim3 grid((Nout + GB_N - 1) / GB_N, (unsigned)((M + GB_M - 1) / GB_M));
    hipLaunchKernelGGL((k_gemm_bf16<bf16>), grid, dim3(256), 0, s, x, (int)M, K, static_cast<const bf16*>(W),
                       Nout, epi);
    return hipGetLastError();
  }
  // fp32: the streaming kernel, one 64-row block per grid row (the weights stay in L2).
  return launch_small<float>(x, (int)M, K, static_cast<const float*>(W), Nout, epi, s);
}

}  // namespace hyf
