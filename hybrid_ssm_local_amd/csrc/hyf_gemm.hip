// bf16 GEMM for K a multiple of 64 (the prefill projections and batched rounds).
//
// Built in its own translation unit with MFMA accumulators in the unified VGPR file
// (-mllvm -amdgpu-mfma-vgpr-form): with accumulation registers the register allocator rotated the
// 128 accumulator registers through copies on every K step.
#include <mutex>
#include <type_traits>

#include "hyf_launch.h"

namespace hyf {

// bf16 GEMM for K a multiple of 64: BM x BN macro tiles (rows x features), K step 64, ST LDS
// stages filled by direct global -> LDS copies.  With NW waves the waves form an (NW/2) x 2 grid:
// wave (wm, wn) owns rows wm*RW .. + RW - 1 (RW = 2 BM / NW) and features wn*BN/2 .. + BN/2 - 1.
// Large products run 256 x 128 tiles with NW = 16 (four waves per SIMD, 32 x 64 per wave, one
// workgroup per CU): the other waves' MFMAs then cover one wave's LDS reads, barrier and copy
// waits.  Products of a few hundred rows (the batched rounds' projections) have too few such tiles
// to fill 256 CUs and take smaller ones (several workgroups per CU).
//
// Per K step a 256 x 128 workgroup does 2*256*128*64 flops against 48 KiB staged, so a CU at the
// MFMA rate needs about 47 B/clk from L2; smaller tiles need more bytes per flop.  Three stages keep
// two K steps of copies in flight while one computes; two workgroups of two stages per CU do the
// same.
//
// LDS operand layout (both operands are K-contiguous rows): row r of a stage is 128 bytes = 8
// chunks of 16 bytes; logical chunk c sits at position c ^ (r & 7), so the 16 lanes of an MFMA
// fragment load (16 rows, one chunk) hit 8 distinct 16-byte bank groups per 8 lanes.  A direct
// copy writes lane l's 16 bytes at base + 16 l, so lane l of a copy covering rows r0 .. r0 + 7
// (r0 a multiple of 8) fetches row r0 + l / 8, logical chunk (l % 8) ^ (l / 8).
constexpr int G2_K = 64;
constexpr int G2_GROUP = 4;  // M tiles per group in the tile order
template <int BM, int BN>
constexpr int g2_stage() { return (BM + BN) * G2_K * 2; }  // bytes per stage (48 KiB at 256 x 128)
// The epilogue stages the fp32 tile ([f][m] or [m][f]) in the stages' LDS, in EH passes of BN / EH
// features each: two passes when the whole tile would not fit in 160 KiB.
template <int BM, int BN>
constexpr int g2_epi_halves() { return BN * (BM + 4) * 4 > 160 * 1024 || BM * (BN + 4) * 4 > 160 * 1024 ? 2 : 1; }
template <int BM, int BN, int ST>
constexpr int g2_lds() {
  constexpr int EN = BN / g2_epi_halves<BM, BN>();
  constexpr int st = ST * g2_stage<BM, BN>(), tr = EN * (BM + 4) * 4, rm = BM * (EN + 4) * 4;
  return st > tr ? (st > rm ? st : rm) : (tr > rm ? tr : rm);
}

// A product of one group of rows (plain launches) carries no row table.
struct NoGroups {};
// Group of product row m (m < M): the last g with m0[g] <= m (empty groups are skipped over).
__device__ __forceinline__ int group_of(const RowGroups& g, int m) {
  int lo = 0, hi = g.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.m0[mid] <= m) lo = mid; else hi = mid - 1;
  }
  return lo;
}
// Store of element (token off of time block blk, feature f) through a time-blocked epilogue.
template <typename T>
__device__ __forceinline__ void epi_store_blk(const Epi& e, int64_t blk, int off, int f, float v) {
  if (f < e.n_split) {
    if (e.out0_f32)
      static_cast<float*>(e.out0)[blk * e.ld0 + (int64_t)f * HYF_TBLK + off] = v;
    else
      static_cast<T*>(e.out0)[blk * e.ld0 + tile_off<T>(f, off)] = from_f32<T>(v);
  } else {
    e.out1[blk * e.ld1 + (int64_t)(f - e.n_split) * HYF_TBLK + off] = v;
  }
}

// Wait until at most n stages of this wave's copies (CP instructions each) are outstanding, n in
// 0..ST-2 (a run-time count near the end of K; vm_wait needs an immediate).
template <int CP, int ST>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (ST >= 4) {
    if (n >= 2) { vm_wait<2 * CP>(); return; }
  }
  if (n >= 1) vm_wait<CP>(); else vm_wait<0>();
}

template <typename TO, int BM, int BN, int NW, int WPE, typename GRP, int ST>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
k_gemm_bf16_tile(RowSrc xs, int M, int K, const bf16* __restrict__ W, int Nout, Epi epi, int tm, int tn,
                 int per_xcd, GRP rows) {
  static_assert(ST >= 2 && ST <= 4, "stages");
  constexpr bool GR = std::is_same<GRP, RowGroups>::value;
  constexpr int G2_M = BM, G2_N = BN, G2_STAGE = g2_stage<BM, BN>();
  constexpr int EH = g2_epi_halves<BM, BN>(), EN = BN / EH;  // epilogue passes, features per pass
  constexpr int BT = BN / 32;  // 16-feature tiles per wave
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0 && BN % 32 == 0 && (2 * BM / NW) % 16 == 0, "tile shape");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // Tile order: workgroup b runs on XCD b % 8; each XCD takes a contiguous range of tiles, walked
  // in groups of G2_GROUP row tiles column by column, so the workgroups an XCD runs together
  // share row and weight slabs in its L2.
  const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (tile >= tm * tn) return;
  const int grp = tile / (G2_GROUP * tn), in_grp = tile % (G2_GROUP * tn);
  const int gm = min(G2_GROUP, tm - grp * G2_GROUP);
  const int mi = grp * G2_GROUP + in_grp % gm, ni = in_grp / gm;
  const int m0 = mi * G2_M, n0 = ni * G2_N;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int i = lane & 15, g = lane >> 4;
  constexpr int NT = 64 * NW;             // threads
  constexpr int RW = G2_M / (NW / 2);     // rows per wave
  constexpr int AT = RW / 16;             // row tiles per wave
  constexpr int CA = G2_M / 8 / NW, CB = G2_N / 8 / NW;  // copies per stage and thread
  const int wm = wave >> 1, wn = wave & 1;
  if (epi.zero && tile == 0)
    for (int z = t; z < epi.n_zero; z += NT) epi.zero[z] = 0;

  // Source rows of this lane's copies: A copy j covers rows 8 (wave + NW j) .. + 7 (j < CA), B
  // copy j rows 8 (wave + NW j) .. + 7 (j < CB); rows past M or Nout repeat the last one (never
  // stored).
  const int lr = lane >> 3, lc = (lane & 7) ^ lr;  // row within the copy, logical chunk
  const char* asrc[CA];
  const char* bsrc[CB];
#pragma unroll
  for (int j = 0; j < CA; ++j) {
    const int m = min(m0 + 8 * (wave + NW * j) + lr, M - 1);
    if constexpr (GR) {
      const int gi = group_of(rows, m);
      const int loc = min(m - rows.m0[gi], rows.cnt[gi] - 1);  // padding rows repeat the group's last row
      asrc[j] = static_cast<const char*>(xs.X1) + ((int64_t)rows.src0[gi] + loc) * K * 2 + 16 * lc;
    } else {
      asrc[j] = static_cast<const char*>(row_ptr(xs, m, K, 2)) + 16 * lc;
    }
  }
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int f = min(n0 + 8 * (wave + NW * j) + lr, Nout - 1);
    bsrc[j] = reinterpret_cast<const char*>(W + (int64_t)f * K) + 16 * lc;
  }
  auto issue = [&](int kt) __attribute__((always_inline)) {
    char* st = smem + (kt % ST) * G2_STAGE;
    const int64_t kb = (int64_t)kt * G2_K * 2;
#pragma unroll
    for (int j = 0; j < CA; ++j) lds_dma16(asrc[j] + kb, st + (wave + NW * j) * 1024);
#pragma unroll
    for (int j = 0; j < CB; ++j) lds_dma16(bsrc[j] + kb, st + G2_M * 128 + (wave + NW * j) * 1024);
  };

  f32x4 acc[AT][BT];
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / G2_K;
#pragma unroll
  for (int k = 0; k < ST - 1; ++k)
    if (k < nk) issue(k);
  // fragment offsets: row r (r & 7 == i & 7), logical chunk c = 4 ks + g at position c ^ (i & 7)
  const int arow = (wm * RW + i) * 128, brow = G2_M * 128 + (wn * (BN / 2) + i) * 128;
  auto frags = [&](const char* st, int ks, bf16x8 (&fa)[AT], bf16x8 (&fb)[BT]) __attribute__((always_inline)) {
    const int co = ((4 * ks + g) ^ (i & 7)) * 16;
#pragma unroll
    for (int a = 0; a < AT; ++a) fa[a] = *reinterpret_cast<const bf16x8*>(st + arow + a * 16 * 128 + co);
#pragma unroll
    for (int b = 0; b < BT; ++b) fb[b] = *reinterpret_cast<const bf16x8*>(st + brow + b * 16 * 128 + co);
  };
  auto mma = [&](const bf16x8 (&fa)[AT], const bf16x8 (&fb)[BT]) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < AT; ++a)
#pragma unroll
      for (int b = 0; b < BT; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
  };
  // Software pipeline over half-steps (32 k values).  Fragments of the next half-step are read
  // while the current half-step's MFMAs run; before a new batch of fragment reads the previous
  // batch is waited on (it has had a whole MFMA batch to land).  The barrier of stage kt + 1 sits
  // between the two half-steps of stage kt: once every wave passes it, stage kt + 1 is in LDS and
  // all reads of stage kt are done, so the copies of stage kt + ST can refill stage kt's buffer
  // (ST - 2 stages stay in flight behind the one that landed).  The barrier is the bare
  // instruction: a __syncthreads() fence would also wait for the copies still in flight.
  auto barrier = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  bf16x8 fa0[AT], fb0[BT], fa1[AT], fb1[BT];
  wait_stages<CA + CB, ST>(min(ST - 2, nk - 1));  // stage 0 landed
  barrier();
  if (ST - 1 < nk) issue(ST - 1);
  frags(smem, 0, fa0, fb0);
  // stage kt: its first half-step's fragments are in fa0/fb0 (read during the previous MFMAs)
  auto first_half = [&](int kt) __attribute__((always_inline)) {
    lgkm_wait0();
    frags(smem + (kt % ST) * G2_STAGE, 1, fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    lgkm_wait0();
  };
  for (int kt = 0; kt + 1 < nk; ++kt) {
    first_half(kt);
    // stage kt + 1 landed once at most the copies of the stages issued after it remain; every
    // wave's reads of stage kt are done, so the copies of stage kt + ST may refill its buffer
    wait_stages<CA + CB, ST>(min(ST - 2, nk - 2 - kt));
    barrier();
    if (kt + ST < nk) issue(kt + ST);
    frags(smem + ((kt + 1) % ST) * G2_STAGE, 0, fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa1, fb1);
    __builtin_amdgcn_sched_barrier(0);
  }
  first_half(nk - 1);
  mma(fa1, fb1);
  __syncthreads();  // the stages are dead: the epilogue reuses LDS

  if (epi.trans) {
    // Time-blocked output: m0 is a multiple of BM, so every run of 8 rows lies in one block.  The
    // fp32 tile is staged as [f][m] (pitch CP floats); each item then writes 8 tokens of one
    // feature: one 16-byte chunk of the tiled layout (out0), or two 16-byte runs of a plain row
    // (out1).
    constexpr int CP = G2_M + 4;
    float* ct = reinterpret_cast<float*>(smem);
    for (int eh = 0; eh < EH; ++eh) {  // feature passes
    if (eh > 0) __syncthreads();  // the previous pass's reads of ct are done
    if (EH == 1 || wn == eh) {
#pragma unroll
      for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int b = 0; b < BT; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            ct[((EH == 1 ? wn * (BN / 2) : 0) + b * 16 + i) * CP + wm * RW + a * 16 + 4 * g + r] = acc[a][b][r];
    }
    __syncthreads();
    for (int it = t; it < EN * (G2_M / 8); it += NT) {
      const int fl = it % EN, m8 = (it / EN) * 8;
      const int f = n0 + eh * EN + fl;
      const int64_t m = (int64_t)m0 + m8;
      if (f >= Nout || m >= M) continue;
      const float* src = ct + fl * CP + m8;
      int64_t blk = m / HYF_TBLK;
      int off = (int)(m % HYF_TBLK);
      bool whole = m + 8 <= M;  // 8 tokens in one block, starting on a multiple of 8
      int gi = 0, loc = 0;
      if constexpr (GR) {
        gi = group_of(rows, (int)m);
        loc = (int)m - rows.m0[gi];
        if (loc >= rows.cnt[gi]) continue;  // padding
        blk = rows.blk0[gi] + loc / HYF_TBLK;
        off = loc % HYF_TBLK;
        whole = loc + 8 <= rows.cnt[gi] && off % 8 == 0;
      }
      if (whole) {
        if (f < epi.n_split && !epi.out0_f32) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = static_cast<bf16>(src[e]);
          *reinterpret_cast<bf16x8*>(static_cast<bf16*>(epi.out0) + blk * epi.ld0 + tile_off<bf16>(f, off)) = v;
        } else {
          float* dst = f < epi.n_split ? static_cast<float*>(epi.out0) + blk * epi.ld0 + (int64_t)f * HYF_TBLK + off
                                       : epi.out1 + blk * epi.ld1 + (int64_t)(f - epi.n_split) * HYF_TBLK + off;
          *reinterpret_cast<f32x4*>(dst) = f32x4{src[0], src[1], src[2], src[3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{src[4], src[5], src[6], src[7]};
        }
      } else if constexpr (GR) {
        // the group's last rows (m0[g] is a multiple of 8, so a run of 8 never spans two groups)
        for (int e = 0; e < 8 && loc + e < rows.cnt[gi]; ++e)
          epi_store_blk<TO>(epi, rows.blk0[gi] + (loc + e) / HYF_TBLK, (loc + e) % HYF_TBLK, f, src[e]);
      } else {
        for (int e = 0; e < 8 && m + e < M; ++e) epi_store<TO>(epi, m + e, f, src[e]);
      }
    }
    }
    return;
  }
  // Row-major output: the fp32 tile is staged as [m][f] (pitch RP floats); each item then writes 8
  // features of one row, as one or two 16-byte stores where the destination allows it.
  constexpr int RP = EN + 4;
  float* ct = reinterpret_cast<float*>(smem);
  for (int eh = 0; eh < EH; ++eh) {  // feature passes
  if (eh > 0) __syncthreads();  // the previous pass's reads of ct are done
  if (EH == 1 || wn == eh) {
#pragma unroll
    for (int a = 0; a < AT; ++a)
#pragma unroll
      for (int b = 0; b < BT; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          ct[(wm * RW + a * 16 + 4 * g + r) * RP + (EH == 1 ? wn * (BN / 2) : 0) + b * 16 + i] = acc[a][b][r];
  }
  __syncthreads();
  for (int it = t; it < G2_M * (EN / 8); it += NT) {
    const int ml = it / (EN / 8), f8 = (it % (EN / 8)) * 8;
    const int64_t m = (int64_t)m0 + ml;
    const int f = n0 + eh * EN + f8;
    if (m >= M || f >= Nout) continue;
    const float* src = ct + ml * RP + f8;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(src), hi = *reinterpret_cast<const f32x4*>(src + 4);
    if (f + 8 <= Nout && (f + 8 <= epi.n_split || f >= epi.n_split)) {
      if (f < epi.n_split && !epi.out0_f32) {
        bf16* dst = static_cast<bf16*>(epi.out0) + m * epi.ld0 + f;
        if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
          bf16x8 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = static_cast<bf16>(lo[e]);
            v[4 + e] = static_cast<bf16>(hi[e]);
          }
          *reinterpret_cast<bf16x8*>(dst) = v;
          continue;
        }
      } else {
        float* dst = f < epi.n_split ? static_cast<float*>(epi.out0) + m * epi.ld0 + f
                                     : epi.out1 + m * epi.ld1 + (f - epi.n_split);
        if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
          *reinterpret_cast<f32x4*>(dst) = lo;
          *reinterpret_cast<f32x4*>(dst + 4) = hi;
          continue;
        }
      }
    }
    for (int e = 0; e < 8 && f + e < Nout; ++e) epi_store<TO>(epi, m, f + e, src[e]);
  }
  }
}

template <int BM, int BN, int NW, int WPE, typename GRP, int ST = 3>
static hipError_t launch_tile(RowSrc x, int M, int K, const bf16* W, int Nout, const Epi& epi, const GRP& grp,
                              hipStream_t s) {
  constexpr int lds = g2_lds<BM, BN, ST>();
  static std::once_flag once;
  static hipError_t set_err = hipSuccess;
  std::call_once(once, [] {
    set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_gemm_bf16_tile<bf16, BM, BN, NW, WPE, GRP, ST>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  });
  if (set_err != hipSuccess) return set_err;
  const int tm = (M + BM - 1) / BM, tn = (Nout + BN - 1) / BN;
  const int per_xcd = (tm * tn + 7) / 8;
  hipLaunchKernelGGL((k_gemm_bf16_tile<bf16, BM, BN, NW, WPE, GRP, ST>), dim3(8 * per_xcd), dim3(64 * NW), lds, s, x,
                     M, K, W, Nout, epi, tm, tn, per_xcd, grp);
  return hipGetLastError();
}

template <typename GRP>
static hipError_t launch_chosen(RowSrc x, int M, int K, const bf16* W, int Nout, const Epi& epi, const GRP& grp,
                                hipStream_t s) {
  auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((Nout + bn - 1) / bn); };
  // fraction of the last wave of tiles (256 CUs, one large tile each) that is busy
  auto fill = [&](int64_t n) { return (double)n / (double)(((n + 255) / 256) * 256); };
  const int64_t t256 = tiles(256, 256);
  if (t256 >= 256 && fill(t256) * 1.12 >= fill(tiles(256, 128)))
    return launch_tile<256, 256, 8, 2, GRP, 2>(x, M, K, W, Nout, epi, grp, s);
  if (tiles(256, 128) >= 384) return launch_tile<256, 128, 16, 4, GRP, 3>(x, M, K, W, Nout, epi, grp, s);
  if (tiles(128, 128) >= 160) return launch_tile<128, 128, 8, 4, GRP, 2>(x, M, K, W, Nout, epi, grp, s);
  if (tiles(128, 64) >= 160) return launch_tile<128, 64, 8, 4>(x, M, K, W, Nout, epi, grp, s);
  return launch_tile<64, 64, 4, 3>(x, M, K, W, Nout, epi, grp, s);
}

// Tile choice, from measured products (bf16, K 2560-5120): 256 x 256 tiles (8 waves of 64 x 128,
// two stages, one workgroup per CU) where there are 256 or more of them and their last wave is not
// much emptier than that of 256 x 128 tiles: about 10% faster than 256 x 128 at 2048 x 2560 x 7968,
// 16384 x 2560 x 7968 and 32768 x 5120 x 5288, but not at 8192 x 2560 x 2720 (352 tiles, 1.4 waves).
// Else 256 x 128 tiles (one workgroup of 16 waves per CU, three stages) once there are 384 or more
// of them; below that the largest of
// 128 x 128 (8 waves, two stages, two workgroups per CU), 128 x 64 (8 waves, two per CU) and
// 64 x 64 (4 waves, three per CU) that still gives 160 or more workgroups, else 64 x 64.  Two
// resident workgroups of two stages each keep as many copies in flight per CU as one of three
// and let one workgroup's MFMAs run through the other's barrier waits: 520 x 2560 x 7968 takes
// 36 us against 47 us for one 128 x 128 workgroup of three stages per CU, and 800 x 2560 x 7968
// 46 us against 51 us for 252 large tiles.  Sixteen waves on the large tile (each a 32 x 64 block)
// beat eight (64 x 64 blocks) by 3-6% from 2048 x 2560 x 7968 up to 32768 x 5120 x 5288.  At
// 512 x 2560 x 2560 the 64 x 64 tiles take 17 us against 28 us for the 80 128 x 128 tiles.
hipError_t launch_gemm256(RowSrc x, int M, int K, const bf16* W, int Nout, const Epi& epi, hipStream_t s) {
  return launch_chosen(x, M, K, W, Nout, epi, NoGroups{}, s);
}

hipError_t launch_gemm_grouped(const bf16* X, const RowGroups& g, int K, const bf16* W, int Nout, const Epi& epi,
                               hipStream_t s) {
  const int M = g.m0[g.n];
  if (M <= 0 || Nout <= 0) return hipSuccess;
  if (K % 64 != 0 || g.n < 1) return hipErrorInvalidValue;
  return launch_chosen(RowSrc{X, X, M}, M, K, W, Nout, epi, g, s);
}

}  // namespace hyf
