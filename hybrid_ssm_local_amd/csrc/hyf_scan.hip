// The recurrent memory's state-only commit scan, one request or many.
//
// Recurrence per head h (plain Mamba-2 / SSD with a scalar decay per head):
//   H <- exp(dt_t * A) H + dt_t * x_t outer B_t,   dt_t = softplus(raw_t + dt_bias), A = -exp(A_log).
// Over a segment of tokens [t0, t1) this folds, exactly, into
//   H_t1 = exp(Lam) H_t0 + sum_t dt_t exp(suf_t) x_t outer B_t,
// where Lam is the segment's total log-decay and suf_t = sum_{t < tau < t1} dt_tau A is the suffix
// log-decay after token t.  Only such sums of log-decays (differences, never ratios of
// exponentials) are exponentiated, so deep decays underflow to 0 instead of becoming 0/0.
//
// The sum over tokens is a per-head contraction (P x tokens) . (tokens x N) on MFMA, with a small
// output (one head's state) and a long reduction: HBM-bound.  x and B come time-blocked and tiled
// (tile_off): tokens in blocks of TB = 128, and inside a block each group of 16 features and run
// of 4 VN tokens (VN = 16 bytes of elements) is one 1 KiB tile holding exactly the 16-byte chunks
// the 64 lanes of one 16x16 MFMA supply, in lane order (16x16x32 bf16: eight k values per lane;
// 16x16x4 fp32: four k values spread over four instructions, the same token order on both
// operands).  So MFMA fragments load straight from global memory into registers with fully
// contiguous 1 KiB wave loads: no LDS staging and no barriers in the main loop.  dt comes
// time-blocked without tiles ([block][feature][TB]).
//
// Work split: each request's chunks are cut into segments (split-K over time); a workgroup owns
// one (segment, head, P-block, N-block), sized so one wave holds the whole output block in
// registers, and its four waves split the segment's tokens again (in 128-byte macro-steps, loads of
// the next macro-step in flight while the current one multiplies).  The waves' partial states meet
// in LDS in a fixed order.  Segment 0 starts from the request's H; a request with one segment
// writes H directly, otherwise k_ssd_combine folds the segment states in order
// (H = P_0, then H = exp(lam_s) H + P_s).  No atomics: the result is deterministic.
//
// With per-token outputs y_t = C_t H_t + D x_t (y-mode) the segments are single blocks:
// k_ssd_blk_state (bf16 heads of up to 128 dimensions) or k_ssd_seg gives every block's own state,
// k_ssd_prefix folds them in order into the state before each block (and the final H), and
// k_ssd_y_mfma (the same bf16 heads) or k_ssd_y computes each block's outputs in the chunk form
// from the state before it.
#include <array>
#include <mutex>
#include <utility>

#include "hyf_launch.h"

namespace hyf {

constexpr int SG_WAVES = 4;                 // waves per workgroup, one per SIMD
constexpr int SG_THREADS = 64 * SG_WAVES;
constexpr int SG_MAX_TILES = 40;            // 16x16 fp32 accumulator tiles per wave (160 registers)
constexpr int SG_MAX_T16 = 8;               // at most 8 tiles along P or along N
constexpr int TB = HYF_TBLK;                // tokens per block of the time-blocked layout

template <typename T>
__device__ __forceinline__ typename Vec16<T>::type ldv(const T* p) {
  return *reinterpret_cast<const typename Vec16<T>::type*>(p);
}

__device__ __forceinline__ int find_request(const ReqTable& rt, int q) {
  int r = 0;
  while (r + 1 < rt.n_req && rt.seg0[r + 1] <= q) ++r;
  return r;
}

template <typename T, int PB16, int NB16>
__global__ void __launch_bounds__(SG_THREADS)
k_ssd_seg(Shape sh, ScanArgs a, ReqTable rt, int npb, int nnb, int n_items, int per_xcd) {
  typedef typename Vec16<T>::type V;
  constexpr int VN = Vec16<T>::n;  // tokens per 16-byte lane load
  constexpr int GT = 4 * VN;       // tokens per load group (four lane groups)
  constexpr int MS = 2 * GT;       // tokens per macro-step: 128 bytes of every feature row
  static_assert(PB16 * NB16 <= SG_MAX_TILES && PB16 <= SG_MAX_T16 && NB16 <= SG_MAX_T16, "tile budget");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* red = reinterpret_cast<float*>(smem);  // [64] pre-pass scratch
  float* wt = red + 64;                         // [segment tokens] per-token weights

  // block b runs on XCD b % 8: consecutive items (the blocks and heads of one segment) share an
  // XCD, so its L2 serves the x rows of a head to all its N-blocks and B to all heads
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (item >= n_items) return;
  const int nh = sh.nh, N = sh.N, P = sh.P;
  const int nb = item % nnb;
  const int pb = (item / nnb) % npb;
  const int h = (item / (nnb * npb)) % nh;
  const int q = item / (nnb * npb * nh);
  const int p0 = pb * PB16 * 16, n0 = nb * NB16 * 16;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int r = find_request(rt, q);
  const int ls = q - rt.seg0[r];
  const int nseg = rt.seg0[r + 1] - rt.seg0[r];
  const int Tr = rt.row0[r + 1] - rt.row0[r];
  const int seg_len = a.seg_tokens;
  const int s_begin = ls * seg_len;
  const int len = min(s_begin + seg_len, Tr) - s_begin;
  const int grp = h / (nh / sh.G);
  const float A = -expf(a.a_log[h]);
  const float bias = a.dt_bias[h];
  // token u of the segment sits in block blk0 + u / TB at offset u % TB (segments start on a
  // block boundary)
  const int64_t blk0 = rt.blk0[r] + s_begin / TB;

  // ---- pre-pass: the per-token weights dt_t exp(suf_t) into LDS.  The segment's raw steps go to
  // LDS in one direct copy (a block's 128 steps of head h are 512 contiguous bytes).  Thread t
  // owns the run of RUN consecutive tokens from t RUN (RUN = 4 run4 with run4 odd, so 16-byte LDS
  // accesses of neighbouring threads fall in different banks).  Forward over the run: dt (kept in
  // LDS in place of the raw step) and the run's log-decay total.  A wave scan and a workgroup
  // scan of the run totals give each run the log-decay of all later tokens; backward over the
  // run, each token's weight replaces its dt.  Tokens past the segment end (up to the end of its
  // last macro-step) get dt = 0, weight 0.
  const int wlen = (len + MS - 1) / MS * MS;
  const int nblk_dt = (len + TB - 1) / TB;
  lds_stage16<SG_THREADS>(nblk_dt * (TB / 4), wt, [&](int i) {
    return a.dt + (blk0 + i / (TB / 4)) * a.dblk + (int64_t)h * TB + 4 * (i % (TB / 4));
  });
  // The request's first segment starts from exp(lam_seg) H: this workgroup's block of H goes to LDS
  // behind the weights (unpitched rows of NB) in the same round trip as the raw steps.
  constexpr int PB = PB16 * 16, NB = NB16 * 16;
  float* Hh = a.h_direct ? a.h_direct + (int64_t)h * P * N
                         : reinterpret_cast<float*>(a.state_pool + (int64_t)rt.slot[r] * sh.st_bytes + sh.st_h) +
                               (int64_t)h * P * N;
  float* hs = wt + (seg_len + MS - 1) / MS * MS;
  if (ls == 0)
    lds_stage16<SG_THREADS>(PB * NB / 4, hs, [&](int i) {
      return Hh + (int64_t)(p0 + i / (NB / 4)) * N + n0 + (i % (NB / 4)) * 4;
    });
  vm_wait<0>();
  __syncthreads();
  const int run4 = ((len + 4 * SG_THREADS - 1) / (4 * SG_THREADS)) | 1;
  const int tk0 = t * 4 * run4;
  float run_tot = 0.f;
#pragma unroll 4
  for (int c = 0; c < run4; ++c) {
    const int tk = tk0 + 4 * c;
    if (tk < wlen) {
      f32x4 d = *reinterpret_cast<const f32x4*>(wt + tk);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d[e] = tk + e < len ? softplus_f(d[e] + bias) : 0.f;
        run_tot += d[e] * A;
      }
      *reinterpret_cast<f32x4*>(wt + tk) = d;
    }
  }
  // exclusive suffix over the runs: later lanes of this wave, then later waves
  float inc = run_tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float v = __shfl_down(inc, o, 64);
    if (lane + o < 64) inc += v;
  }
  if (lane == 0) red[wave] = inc;
  __syncthreads();
  float suf = __shfl_down(inc, 1, 64);
  if (lane == 63) suf = 0.f;
  float lam_seg = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < SG_WAVES; ++w2) {
    if (w2 > wave) suf += red[w2];
    lam_seg += red[w2];
  }
#pragma unroll 4
  for (int c = run4 - 1; c >= 0; --c) {
    const int tk = tk0 + 4 * c;
    if (tk < wlen) {
      f32x4 d = *reinterpret_cast<const f32x4*>(wt + tk);
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        const float w = d[e] * __expf(suf);  // suf <= 0
        suf += d[e] * A;
        d[e] = w;
      }
      *reinterpret_cast<f32x4*>(wt + tk) = d;
    }
  }

  // ---- accumulators.  Tile (pt, nt), lane (li, lg), register rr holds state row
  // p0 + 16 pt + 4 lg + rr, column n0 + 16 nt + li (the MFMA output layout).  Wave 0 of the
  // request's first segment starts from exp(lam_seg) H (staged above); every other accumulator
  // starts at 0.
  constexpr int RP = NB + 4;
  __syncthreads();  // weights complete
  f32x4 acc[PB16][NB16];
#pragma unroll
  for (int pt = 0; pt < PB16; ++pt)
#pragma unroll
    for (int nt = 0; nt < NB16; ++nt) acc[pt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (ls == 0 && wave == 0) {
    const float d0 = expf(lam_seg);
#pragma unroll
    for (int pt = 0; pt < PB16; ++pt)
#pragma unroll
      for (int nt = 0; nt < NB16; ++nt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[pt][nt][rr] = d0 * hs[(pt * 16 + 4 * lg + rr) * NB + nt * 16 + li];
  }

  // ---- operand loads.  With the tiled layout the 16-byte chunk lane l brings for an MFMA sits at
  // byte 16 l of a 1 KiB tile, so a load is a scalar base (the segment's first block, in a buffer
  // resource), a scalar offset (block, feature group, token run) and the lane offset 16 l.  The
  // segment's blocks span less than 2 GiB, so every offset fits in 32 bits; the resource's size
  // also turns any read past the segment's last block into zeros.
  constexpr int NJ = TB / GT;  // token runs (tiles) per feature group and block
  const int nblk_seg = (len + TB - 1) / TB;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(static_cast<const T*>(a.x) + blk0 * a.xblk), 0, (int)(nblk_seg * a.xblk * sizeof(T)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(static_cast<const T*>(a.B) + blk0 * a.bblk), 0, (int)(nblk_seg * a.bblk * sizeof(T)), 0x00020000);
  const int fga = (h * P + p0) / 16, fgb = (grp * N + n0) / 16;  // first feature group of x, B
  const int loff = lane * 16;
  auto load = [&](V (&fa)[PB16][2], V (&fb)[NB16][2], int m) __attribute__((always_inline)) {
    const int u = m * MS;
    const int j0 = (u % TB) / GT;
    const int sx = (int)(((u / TB) * a.xblk + ((int64_t)fga * NJ + j0) * 64 * VN) * sizeof(T));
    const int sb = (int)(((u / TB) * a.bblk + ((int64_t)fgb * NJ + j0) * 64 * VN) * sizeof(T));
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int pt = 0; pt < PB16; ++pt)
        fa[pt][g] = __builtin_bit_cast(
            V, __builtin_amdgcn_raw_buffer_load_b128(rx, loff, sx + (pt * NJ + g) * 1024, 0));
#pragma unroll
      for (int nt = 0; nt < NB16; ++nt)
        fb[nt][g] = __builtin_bit_cast(
            V, __builtin_amdgcn_raw_buffer_load_b128(rb, loff, sb + (nt * NJ + g) * 1024, 0));
    }
  };

  // ---- main loop.  Wave w takes macro-steps [w M / 4, (w + 1) M / 4) of the segment.  In a
  // macro-step, for load group g = 0, 1, lane (li, lg) holds the VN tokens
  // u + g GT + lg VN .. + VN - 1 of x row p0 + 16 pt + li (every pt) and of B row n0 + 16 nt + li
  // (every nt); x is scaled by the tokens' weights and the pair enters the MFMAs.
  const int M = wlen / MS;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // uniform: keeps offsets scalar
  const int m_lo = wave_u * M / SG_WAVES, m_hi = (wave_u + 1) * M / SG_WAVES;
  auto compute = [&](V (&fa)[PB16][2], V (&fb)[NB16][2], int m) __attribute__((always_inline)) {
    const int u = m * MS;
    const bool tail = u + MS > len;  // the segment's last macro-step: mask tokens past its end
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int tb = u + g * GT + lg * VN;  // first token of this lane's VN tokens
      float w[VN];
#pragma unroll
      for (int e4 = 0; e4 < VN; e4 += 4) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(wt + tb + e4);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e4 + e] = w4[e];
      }
      V sa[PB16];
#pragma unroll
      for (int pt = 0; pt < PB16; ++pt)
#pragma unroll
        for (int e = 0; e < VN; ++e) sa[pt][e] = from_f32<T>(to_f32(fa[pt][g][e]) * w[e]);
      if (tail) {
        // the inputs past the end hold anything (NaN included): zero both operands there
#pragma unroll
        for (int e = 0; e < VN; ++e) {
          if (tb + e >= len) {
#pragma unroll
            for (int pt = 0; pt < PB16; ++pt) sa[pt][e] = from_f32<T>(0.f);
#pragma unroll
            for (int nt = 0; nt < NB16; ++nt) fb[nt][g][e] = from_f32<T>(0.f);
          }
        }
      }
      if constexpr (VN == 8) {
#pragma unroll
        for (int pt = 0; pt < PB16; ++pt)
#pragma unroll
          for (int nt = 0; nt < NB16; ++nt) acc[pt][nt] = Mfma16<T>::mma(sa[pt], fb[nt][g], acc[pt][nt]);
      } else {
        // fp32: k index lg of instruction j is token tb + j on both operands
#pragma unroll
        for (int j = 0; j < VN; ++j)
#pragma unroll
          for (int pt = 0; pt < PB16; ++pt)
#pragma unroll
            for (int nt = 0; nt < NB16; ++nt) acc[pt][nt] = Mfma16<T>::mma(sa[pt][j], fb[nt][g][j], acc[pt][nt]);
      }
    }
  };

  if (m_lo < m_hi) {
    V fa0[PB16][2], fb0[NB16][2], fa1[PB16][2], fb1[NB16][2];
    load(fa0, fb0, m_lo);
    for (int m = m_lo; m < m_hi; m += 2) {
      // the next macro-step's loads go out before this one's MFMAs (a clamped index repeats the
      // last macro-step's loads at the end instead of branching around them)
      load(fa1, fb1, min(m + 1, m_hi - 1));
      compute(fa0, fb0, m);
      if (m + 1 >= m_hi) break;
      load(fa0, fb0, min(m + 2, m_hi - 1));
      compute(fa1, fb1, m + 1);
    }
  }

  // ---- the four waves' states meet in LDS (weights and staged H are dead now), row-major with
  // row pitch RP (the 4 row groups of a tile land in different banks): (w0 + w2) + (w1 + w3),
  // written as 16-byte runs by all threads.
  __syncthreads();
  float* slot = reinterpret_cast<float*>(smem);
  auto put = [&](int sl) __attribute__((always_inline)) {
#pragma unroll
    for (int pt = 0; pt < PB16; ++pt)
#pragma unroll
      for (int nt = 0; nt < NB16; ++nt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) slot[(sl * PB + pt * 16 + 4 * lg + rr) * RP + nt * 16 + li] = acc[pt][nt][rr];
  };
  auto add = [&](int sl) __attribute__((always_inline)) {
#pragma unroll
    for (int pt = 0; pt < PB16; ++pt)
#pragma unroll
      for (int nt = 0; nt < NB16; ++nt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[pt][nt][rr] += slot[(sl * PB + pt * 16 + 4 * lg + rr) * RP + nt * 16 + li];
  };
  if (wave >= 2) put(wave - 2);
  __syncthreads();
  if (wave < 2) add(wave);
  __syncthreads();
  if (wave < 2) put(wave);
  __syncthreads();

  float* dst;
  if (nseg == 1 && !a.y_mode) {
    dst = Hh;
  } else {
    dst = a.part + ((int64_t)q * nh + h) * P * N;
    if (pb == 0 && nb == 0 && t == 0) a.lam[(int64_t)q * nh + h] = lam_seg;
  }
  for (int idx = t; idx < PB * NB / 4; idx += SG_THREADS) {
    const int p = idx / (NB / 4), n = (idx % (NB / 4)) * 4;
    const f32x4 v = *reinterpret_cast<const f32x4*>(slot + p * RP + n) + *reinterpret_cast<const f32x4*>(slot + (PB + p) * RP + n);
    *reinterpret_cast<f32x4*>(dst + (int64_t)(p0 + p) * N + n0 + n) = v;
  }
}

// Folds the segment states of requests with more than one segment, in segment order.
__global__ void __launch_bounds__(256) k_ssd_combine(Shape sh, ScanArgs a, ReqTable rt) {
  const int nh = sh.nh;
  const int r = blockIdx.x / nh, h = blockIdx.x % nh;
  const int s0 = rt.seg0[r], s1 = rt.seg0[r + 1];
  if (s1 - s0 <= 1) return;
  const int64_t PN = (int64_t)sh.P * sh.N;
  const int64_t e = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
  if (e >= PN) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(a.part + ((int64_t)s0 * nh + h) * PN + e);
  for (int s = s0 + 1; s < s1; ++s) {
    const float d = expf(a.lam[(int64_t)s * nh + h]);
    const f32x4 p = *reinterpret_cast<const f32x4*>(a.part + ((int64_t)s * nh + h) * PN + e);
    acc = acc * d + p;
  }
  float* Hh = a.h_direct ? a.h_direct + (int64_t)h * PN
                         : reinterpret_cast<float*>(a.state_pool + (int64_t)rt.slot[r] * sh.st_bytes + sh.st_h) +
                               (int64_t)h * PN;
  *reinterpret_cast<f32x4*>(Hh + e) = acc;
}

// y-mode fold: per (request, head), the state before every segment replaces that segment's
// partial (segment 0 starts from H), and H becomes the state after the last segment.
__global__ void __launch_bounds__(256) k_ssd_prefix(Shape sh, ScanArgs a, ReqTable rt) {
  const int nh = sh.nh;
  const int r = blockIdx.x / nh, h = blockIdx.x % nh;
  const int s0 = rt.seg0[r], s1 = rt.seg0[r + 1];
  if (s1 == s0) return;
  const int64_t PN = (int64_t)sh.P * sh.N;
  const int64_t e = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
  if (e >= PN) return;
  float* Hh = a.h_direct ? a.h_direct + (int64_t)h * PN
                         : reinterpret_cast<float*>(a.state_pool + (int64_t)rt.slot[r] * sh.st_bytes + sh.st_h) +
                               (int64_t)h * PN;
  f32x4* p0 = reinterpret_cast<f32x4*>(a.part + ((int64_t)s0 * nh + h) * PN + e);
  f32x4 acc = *p0;  // segment 0's partial includes exp(lam_0) H
  *p0 = *reinterpret_cast<const f32x4*>(Hh + e);
  for (int s = s0 + 1; s < s1; ++s) {
    const float d = expf(a.lam[(int64_t)s * nh + h]);
    f32x4* ps = reinterpret_cast<f32x4*>(a.part + ((int64_t)s * nh + h) * PN + e);
    const f32x4 p = *ps;
    *ps = acc;
    acc = acc * d + p;
  }
  *reinterpret_cast<f32x4*>(Hh + e) = acc;
}

// y-mode outputs, the chunked form of the recurrence: per (block of TB tokens, head), with H0 the
// state before the block, a_s = dt_s A and cum_t = a_0 + ... + a_t,
//   y_t = sum_{s <= t} exp(cum_t - cum_s) dt_s (C_t . B_s) x_s + exp(cum_t) H0 C_t + D x_t.
// The block's x (this head), B and C are staged in LDS in their tiled layout (three contiguous
// copies); every product runs on fp32 16x16x4 MFMAs with operands gathered element-wise from LDS
// (exact products of the stored values):
//   G^T[s][t] = sum_n B[s][n] C[t][n] for a 16 x 16 (s, t) tile, whose output register r of lane
//   (li, lg) is G[t0 + li][s0 + 4 lg + r]: masked and scaled into M[t][s], it is already the A
//   operand of Y += M X (instruction j contracts s0 + 4 lg + j);
//   the state term sum_n C[t][n] H0[p][n] with H0 read from global memory, four columns a load.
// Wave w takes the output row tiles w and 7 - w (the causal sums then cost each wave the same).
template <typename T, int MAXT>
__global__ void __launch_bounds__(256) k_ssd_y(Shape sh, ScanArgs a, ReqTable rt, int h0_lds) {
  constexpr int VN = Vec16<T>::n;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nh = sh.nh, P = sh.P, N = sh.N;
  const int h = blockIdx.x % nh, q = blockIdx.x / nh;
  const int r = find_request(rt, q);
  const int ls = q - rt.seg0[r];
  const int Tr = rt.row0[r + 1] - rt.row0[r];
  const int s_begin = ls * TB;
  const int len = min(TB, Tr - s_begin);
  const int64_t blk = rt.blk0[r] + ls;  // y-mode segments are single blocks
  const int grp = h / (nh / sh.G);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int li = lane & 15, lg = lane >> 4;
  T* xs = reinterpret_cast<T*>(smem);  // tiled [P][TB]
  T* bs = xs + P * TB;                 // tiled [N][TB]
  T* cs = bs + N * TB;                 // tiled [N][TB]
  float* dts = reinterpret_cast<float*>(cs + N * TB);  // [TB] raw steps, then dt
  float* cum = dts + TB;                               // [TB]
  // the 16-feature groups of a block are contiguous: features f0 .. f0 + F of a block start at
  // element f0 TB of it
  const T* gx = static_cast<const T*>(a.x) + blk * a.xblk + (int64_t)h * P * TB;
  const T* gb = static_cast<const T*>(a.B) + blk * a.bblk + (int64_t)grp * N * TB;
  const T* gc = static_cast<const T*>(a.C) + blk * a.cblk + (int64_t)grp * N * TB;
  const float* gd = a.dt + blk * a.dblk + (int64_t)h * TB;
  lds_stage16<256>(P * TB / VN, xs, [&](int i) { return gx + (int64_t)i * VN; });
  lds_stage16<256>(N * TB / VN, bs, [&](int i) { return gb + (int64_t)i * VN; });
  lds_stage16<256>(N * TB / VN, cs, [&](int i) { return gc + (int64_t)i * VN; });
  lds_stage16<256>(TB / 4, dts, [&](int i) { return gd + 4 * i; });
  // the state before the block, when it fits: [P][N] fp32, 16-byte chunk c of row p at position
  // c ^ (p & 7) (the 16 rows of an MFMA operand load fall in 8 different bank groups)
  float* h0s = cum + TB;
  const float* H0 = a.part + ((int64_t)q * nh + h) * P * N;  // state before the block
  const int cpr = N / 4;
  if (h0_lds)
    lds_stage16<256>(P * cpr, h0s, [&](int i) {
      const int p = i / cpr, pc = i % cpr;
      return H0 + (int64_t)p * N + 4 * (pc ^ (p & 7));
    });
  vm_wait<0>();
  __syncthreads();
  if (wave == 0) {
    // dt and the inclusive prefix of a = dt A (tokens past len: dt = 0)
    const float A = -expf(a.a_log[h]), bias = a.dt_bias[h];
    const int u0 = 2 * lane;
    const float d0 = u0 < len ? softplus_f(dts[u0] + bias) : 0.f;
    const float d1 = u0 + 1 < len ? softplus_f(dts[u0 + 1] + bias) : 0.f;
    const float a0 = d0 * A, a1 = d1 * A;
    float inc = a0 + a1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    const float ex = inc - (a0 + a1);
    cum[u0] = ex + a0;
    cum[u0 + 1] = inc;
    dts[u0] = d0;
    dts[u0 + 1] = d1;
  }
  __syncthreads();

  const int ntp = P / 16;
  const float D = a.d_skip[h];
  T* yout = static_cast<T*>(a.y) + ((int64_t)rt.row0[r] + s_begin) * nh * P + (int64_t)h * P;
  for (int pass = 0; pass < 2; ++pass) {
    const int tt = pass ? TB / 16 - 1 - wave : wave;
    const int t0 = 16 * tt;
    if (t0 >= len) continue;
    f32x4 y[MAXT], yi[MAXT];
#pragma unroll
    for (int i = 0; i < MAXT; ++i) y[i] = yi[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int st = 0; st <= tt && 16 * st < len; ++st) {
      const int s0 = 16 * st;
      // four independent chains over n (reads of a group of 64 columns issue together)
      f32x4 g4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) g4[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int n0 = 0; n0 < N; n0 += 64) {
        float bv[4][4], cv[4][4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = min(n0 + 16 * k + 4 * lg + j, N - 1);
            bv[k][j] = to_f32(bs[tile_off<T>(n, s0 + li)]);
            cv[k][j] = to_f32(cs[tile_off<T>(n, t0 + li)]);
          }
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (n0 + 16 * k < N)
#pragma unroll
            for (int j = 0; j < 4; ++j) g4[k] = Mfma16<float>::mma(bv[k][j], cv[k][j], g4[k]);
      }
      const f32x4 g = (g4[0] + g4[1]) + (g4[2] + g4[3]);
      float mv[4];
      const int tq = t0 + li;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int sq = s0 + 4 * lg + rr;
        mv[rr] = sq <= tq && sq < len ? g[rr] * expf(cum[tq] - cum[sq]) * dts[sq] : 0.f;
      }
#pragma unroll
      for (int pt = 0; pt < MAXT; ++pt) {
        if (pt < ntp) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int sq = s0 + 4 * lg + j;
            const float xv = sq < len ? to_f32(xs[tile_off<T>(16 * pt + li, sq)]) : 0.f;
            y[pt] = Mfma16<float>::mma(mv[j], xv, y[pt]);
          }
        }
      }
    }
    // state term: yi[t][p] = sum_n C[t][n] H0[p][n]
#pragma unroll 4
    for (int n0 = 0; n0 < N; n0 += 16) {
      float cv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) cv[j] = to_f32(cs[tile_off<T>(n0 + 4 * lg + j, t0 + li)]);
#pragma unroll
      for (int pt = 0; pt < MAXT; ++pt) {
        if (pt < ntp) {
          const int p = 16 * pt + li;
          const f32x4 hv = h0_lds ? *reinterpret_cast<const f32x4*>(h0s + p * N + 4 * (((n0 >> 2) + lg) ^ (li & 7)))
                                  : *reinterpret_cast<const f32x4*>(H0 + (int64_t)p * N + n0 + 4 * lg);
#pragma unroll
          for (int j = 0; j < 4; ++j) yi[pt] = Mfma16<float>::mma(cv[j], hv[j], yi[pt]);
        }
      }
    }
    // lane (li, lg) register rr: token t0 + 4 lg + rr, column 16 pt + li
#pragma unroll
    for (int pt = 0; pt < MAXT; ++pt) {
      if (pt < ntp) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int tq = t0 + 4 * lg + rr;
          if (tq < len) {
            const int p = 16 * pt + li;
            const float v = y[pt][rr] + expf(cum[tq]) * yi[pt][rr] + D * to_f32(xs[tile_off<T>(p, tq)]);
            yout[(int64_t)tq * nh * P + p] = from_f32<T>(v);
          }
        }
      }
    }
  }
}

// y-mode block states on bf16 matrix cores: one workgroup per (block, head) forms the block's own
// contribution to the state, S[p][n] = sum_t w_t x_t[p] B_t[n] with w_t = dt_t exp(suf_t) and suf_t
// the log-decay of the block's tokens after t (a request's first block adds exp(Lam) H, Lam the
// block's total log-decay, which goes to lam).  The transposed product S^T = (w B)^T x^T is one
// 16x16x32 MFMA chain per 16 x 16 output tile whose operands are the tiled layouts as they stand:
// lane (i, g) of tile (fg, j) of B holds feature 16 fg + i at tokens 32 j + 8 g .. + 7 (the A
// operand, scaled by the weights and split into two bf16 terms, hi and lo), and lane (i, g) of
// tile (pt, j) of x holds feature 16 pt + i at the same tokens (the B operand).  Accumulator
// register r of lane (i, g) is S[16 pt + i][16 fg + 4 g + r]: one 16-byte store per lane and tile.
// Wave w owns the feature groups w, w + 4, ...  Tokens past the block's length are zeroed on both
// operands (their stored values may be anything).
template <int PB>
__global__ void __launch_bounds__(256) k_ssd_blk_state(Shape sh, ScanArgs a, ReqTable rt) {
  constexpr int NJ = TB / 32;  // 32-token runs of a block
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ float s_lam;
  const int nh = sh.nh, P = 16 * PB, N = sh.N, NFG = N / 16;
  const int h = blockIdx.x % nh, q = blockIdx.x / nh;
  const int r = find_request(rt, q);
  const int ls = q - rt.seg0[r];
  const int Tr = rt.row0[r + 1] - rt.row0[r];
  const int len = min(TB, Tr - ls * TB);
  const int64_t blk = rt.blk0[r] + ls;  // y-mode segments are single blocks
  const int grp = h / (nh / sh.G);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int li = lane & 15, g = lane >> 4;
  char* xs = smem;                                           // x: PB x NJ tiles of 1 KiB
  char* bs = smem + PB * NJ * 1024;                          // B: NFG x NJ tiles
  float* wt = reinterpret_cast<float*>(bs + NFG * NJ * 1024);  // [TB] raw steps, then weights
  const bf16* gx = static_cast<const bf16*>(a.x) + blk * a.xblk + (int64_t)h * P * TB;
  const bf16* gb = static_cast<const bf16*>(a.B) + blk * a.bblk + (int64_t)grp * N * TB;
  const float* gd = a.dt + blk * a.dblk + (int64_t)h * TB;
  lds_stage16<256>(P * TB / 8, xs, [&](int i) { return gx + (int64_t)i * 8; });
  lds_stage16<256>(N * TB / 8, bs, [&](int i) { return gb + (int64_t)i * 8; });
  lds_stage16<256>(TB / 4, wt, [&](int i) { return gd + 4 * i; });
  vm_wait<0>();
  __syncthreads();
  if (wave == 0) {
    // lane l holds tokens 2 l, 2 l + 1; a = dt A (0 past len); the log-decay after a token is a
    // suffix sum over the lanes (a sum of later log-decays, never a difference of prefixes)
    const float A = -expf(a.a_log[h]), bias = a.dt_bias[h];
    const int u0 = 2 * lane;
    const float d0 = u0 < len ? softplus_f(wt[u0] + bias) : 0.f;
    const float d1 = u0 + 1 < len ? softplus_f(wt[u0 + 1] + bias) : 0.f;
    const float a0 = d0 * A, a1 = d1 * A;
    float inc = a0 + a1;  // sum over this lane and the lanes after it
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float v = __shfl_down(inc, o, 64);
      if (lane + o < 64) inc += v;
    }
    const float after = inc - (a0 + a1);  // tokens after 2 l + 1
    wt[u0] = d0 * expf(after + a1);
    wt[u0 + 1] = d1 * expf(after);
    if (lane == 0) s_lam = inc;
  }
  __syncthreads();
  const float lam = s_lam;
  const float el = expf(lam);
  const float* Hh = a.h_direct ? a.h_direct + (int64_t)h * P * N
                               : reinterpret_cast<const float*>(a.state_pool + (int64_t)rt.slot[r] * sh.st_bytes +
                                                                sh.st_h) + (int64_t)h * P * N;
  float* dst = a.part + ((int64_t)q * nh + h) * P * N;
  for (int fg = wave; fg < NFG; fg += 4) {
    bf16x8 ah[NJ], al[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(bs + (fg * NJ + j) * 1024 + 16 * lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = 32 * j + 8 * g + e;
        const float v = tok < len ? wt[tok] * static_cast<float>(b[e]) : 0.f;
        const bf16 hb = static_cast<bf16>(v);
        ah[j][e] = hb;
        al[j][e] = static_cast<bf16>(v - static_cast<float>(hb));
      }
    }
#pragma unroll
    for (int pt = 0; pt < PB; ++pt) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        bf16x8 xv = *reinterpret_cast<const bf16x8*>(xs + (pt * NJ + j) * 1024 + 16 * lane);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (32 * j + 8 * g + e >= len) xv[e] = static_cast<bf16>(0.f);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[j], xv, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[j], xv, acc, 0, 0, 0);
      }
      const int64_t o = (int64_t)(16 * pt + li) * N + 16 * fg + 4 * g;
      if (ls == 0) acc += el * *reinterpret_cast<const f32x4*>(Hh + o);
      *reinterpret_cast<f32x4*>(dst + o) = acc;
    }
  }
  if (t == 0) a.lam[(int64_t)q * nh + h] = lam;
}

// y-mode outputs of a bf16 block on bf16 matrix cores (16x16x16, fp32 sums), the same chunked
// form as k_ssd_y, with eight waves: wave w owns output tile w (tokens 16 w .. 16 w + 15).
// B and C of the block go to LDS in their tiled layout and are turned in place, one 1 KiB tile (16
// features x 32 tokens) at a time, into token-major 16 x 16 blocks: the tile is the A operand of a
// 16x16x32 product with a 0/1 matrix I_h (h: which 16 of its 32 tokens), D = A I_h, whose
// accumulator layout (lane (i, g): features 4 g .. + 3 of token i) is the operand layout of a
// product contracting over features; written back as 512-byte halves of the same tile, so the
// turn needs no other buffer.  Then per input tile s <= t:
//   G^T[s][t] = sum_n B[s][n] C[t][n]      (A: B block of s, B: C block of t, exact bf16 products);
//   its accumulator (lane (i, g): token t0 + i, tokens s0 + 4 g + r) masked and scaled into
//   M[t][s] = exp(cum_t - cum_s) dt_s G[t][s] is the A operand of Y += M X, M entering as two bf16
//   terms (hi, lo) and X as 8-byte pieces of the tiled x read from global memory one step ahead;
// and the state term sum_n C[t][n] H0[p][n], H0 (fp32, global, one feature group ahead up to 96
// head dimensions) as two bf16 terms.  The x pieces of the diagonal step (s = t) are the x_t the
// skip term D x_t needs.
// Inputs past the block's length hold anything: B and C there are zeroed before the turn (a product
// with I_h sums every token of the run), their scores are replaced by 0 and their x pieces read as 0.
template <int PB>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
k_ssd_y_mfma(Shape sh, ScanArgs a, ReqTable rt) {
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  constexpr int NJ = TB / 32;  // 32-token runs of a block
  constexpr int NWV = TB / 16;  // waves: one per 16-token tile
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nh = sh.nh, P = 16 * PB, N = sh.N, NFG = N / 16;
  const int h = blockIdx.x % nh, q = blockIdx.x / nh;
  const int r = find_request(rt, q);
  const int ls = q - rt.seg0[r];
  const int Tr = rt.row0[r + 1] - rt.row0[r];
  const int s_begin = ls * TB;
  const int len = min(TB, Tr - s_begin);
  const int64_t blk = rt.blk0[r] + ls;  // y-mode segments are single blocks
  const int grp = h / (nh / sh.G);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int li = lane & 15, g = lane >> 4;
  char* bs = smem;                   // B: NFG x NJ tiles of 1 KiB
  char* cs = smem + NFG * NJ * 1024;  // C, the same
  float* dts = reinterpret_cast<float*>(cs + NFG * NJ * 1024);  // [TB] raw steps, then dt
  float* cum = dts + TB;                                         // [TB]
  const bf16* gx = static_cast<const bf16*>(a.x) + blk * a.xblk + (int64_t)h * P * TB;
  const bf16* gb = static_cast<const bf16*>(a.B) + blk * a.bblk + (int64_t)grp * N * TB;
  const bf16* gc = static_cast<const bf16*>(a.C) + blk * a.cblk + (int64_t)grp * N * TB;
  const float* gd = a.dt + blk * a.dblk + (int64_t)h * TB;
  const float* H0 = a.part + ((int64_t)q * nh + h) * P * N;  // state before the block
  lds_stage16<512>(N * TB / 8, bs, [&](int i) { return gb + (int64_t)i * 8; });
  lds_stage16<512>(N * TB / 8, cs, [&](int i) { return gc + (int64_t)i * 8; });
  lds_stage16<512>(TB / 4, dts, [&](int i) { return gd + 4 * i; });
  // this wave's output tile, its first x pieces and H0's first feature group, in flight with the
  // staging (X[s0 + 4 g .. + 3][16 pt + li]: half of a 16-byte chunk of the tiled x)
  const int t0 = 16 * wave;
  auto load_x = [&](int s0, s16x4* xv) {
    const int tok = s0 + 4 * g;
    const int64_t xo = ((tok / 32) * 64 + ((tok % 32) / 8) * 16 + li) * 8 + tok % 8;
#pragma unroll
    for (int pt = 0; pt < PB; ++pt) xv[pt] = *reinterpret_cast<const s16x4*>(gx + (int64_t)pt * NJ * 64 * 8 + xo);
  };
  auto load_h = [&](int fg, f32x4* hv) {
#pragma unroll
    for (int pt = 0; pt < PB; ++pt)
      hv[pt] = *reinterpret_cast<const f32x4*>(H0 + (int64_t)(16 * pt + li) * N + 16 * fg + 4 * g);
  };
  s16x4 xa[PB];
  f32x4 hc[PB];
  if (t0 < len) {
    load_x(0, xa);
    load_h(0, hc);
  }
  vm_wait<0>();
  __syncthreads();
  // ---- turn B and C token-major (each wave its own tiles, in place) and form dt and cum
  {
    bf16x8 id[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) id[hh][e] = static_cast<bf16>(8 * g + e == 16 * hh + li ? 1.f : 0.f);
    for (int tile = wave; tile < 2 * NFG * NJ; tile += NWV) {
      char* tb = (tile < NFG * NJ ? bs : cs) + (tile % (NFG * NJ)) * 1024;
      bf16x8 v = *reinterpret_cast<const bf16x8*>(tb + 16 * lane);
      // tokens past the length may hold NaN or infinity, which a 0 of I_h would not cancel
      const int tok = 32 * (tile % NJ) + 8 * g;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (tok + e >= len) v[e] = static_cast<bf16>(0.f);
      f32x4 d[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        d[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, id[hh], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        s16x4 o;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) o[rr] = __builtin_bit_cast(short, static_cast<bf16>(d[hh][rr]));  // exact
        *reinterpret_cast<s16x4*>(tb + 512 * hh + 8 * lane) = o;
      }
    }
  }
  if (wave == 0) {
    // dt and the inclusive prefix of a = dt A (tokens past len: dt = 0)
    const float A = -expf(a.a_log[h]), bias = a.dt_bias[h];
    const int u0 = 2 * lane;
    const float d0 = u0 < len ? softplus_f(dts[u0] + bias) : 0.f;
    const float d1 = u0 + 1 < len ? softplus_f(dts[u0 + 1] + bias) : 0.f;
    const float a0 = d0 * A, a1 = d1 * A;
    float inc = a0 + a1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    const float ex = inc - (a0 + a1);
    cum[u0] = ex + a0;
    cum[u0 + 1] = inc;
    dts[u0] = d0;
    dts[u0 + 1] = d1;
  }
  __syncthreads();
  if (t0 >= len) return;  // uniform; no barrier follows

  // 16 x 16 token-major block (token tile tt, feature group fg) of B or C: lane (i, g) reads token
  // 16 tt + i, features 16 fg + 4 g .. + 3
  auto blk8 = [&](const char* base, int tt, int fg) {
    return *reinterpret_cast<const s16x4*>(base + (fg * NJ + tt / 2) * 1024 + (tt % 2) * 512 + 8 * lane);
  };
  const int tt = wave;
  f32x4 y[PB], ys[PB];
#pragma unroll
  for (int pt = 0; pt < PB; ++pt) y[pt] = ys[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // state term: ys[t][p] = sum_n C[t][n] H0[p][n], H0 as two bf16 terms
  constexpr bool HPF = PB <= 6;  // H0 one feature group ahead while it fits the registers
  for (int fg = 0; fg < NFG; ++fg) {
    f32x4 hn[PB];
    if (HPF && fg + 1 < NFG) load_h(fg + 1, hn);
    if (!HPF && fg > 0) load_h(fg, hc);
    const s16x4 cv = blk8(cs, tt, fg);
#pragma unroll
    for (int pt = 0; pt < PB; ++pt) {
      s16x4 hh, hl;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const bf16 hb = static_cast<bf16>(hc[pt][rr]);
        hh[rr] = __builtin_bit_cast(short, hb);
        hl[rr] = __builtin_bit_cast(short, static_cast<bf16>(hc[pt][rr] - static_cast<float>(hb)));
      }
      ys[pt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cv, hh, ys[pt], 0, 0, 0);
      ys[pt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cv, hl, ys[pt], 0, 0, 0);
    }
    if (HPF && fg + 1 < NFG)
#pragma unroll
      for (int pt = 0; pt < PB; ++pt) hc[pt] = hn[pt];
  }
  const float ct = cum[t0 + li];
  for (int st = 0; st <= tt; ++st) {
    const int s0 = 16 * st;
    s16x4 xn[PB];
    if (st < tt) load_x(s0 + 16, xn);  // the next step's pieces (the diagonal step is always inside len)
    f32x4 gt = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int fg = 0; fg < NFG; ++fg)
      gt = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(blk8(bs, st, fg), blk8(cs, tt, fg), gt, 0, 0, 0);
    // lane (li, g) register rr: G[t0 + li][s0 + 4 g + rr]
    s16x4 mh, ml;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int sq = s0 + 4 * g + rr;
      const float m = sq <= t0 + li && sq < len ? gt[rr] * expf(ct - cum[sq]) * dts[sq] : 0.f;
      const bf16 hb = static_cast<bf16>(m);
      mh[rr] = __builtin_bit_cast(short, hb);
      ml[rr] = __builtin_bit_cast(short, static_cast<bf16>(m - static_cast<float>(hb)));
    }
    const int tok = s0 + 4 * g;
#pragma unroll
    for (int pt = 0; pt < PB; ++pt) {
      s16x4 xv = xa[pt];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (tok + rr >= len) xv[rr] = 0;  // x past the block's length may hold anything
      y[pt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mh, xv, y[pt], 0, 0, 0);
      y[pt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ml, xv, y[pt], 0, 0, 0);
    }
    if (st < tt)
#pragma unroll
      for (int pt = 0; pt < PB; ++pt) xa[pt] = xn[pt];
  }
  // lane (li, g) register rr: token t0 + 4 g + rr, column 16 pt + li; xa holds x at the same places
  const float D = a.d_skip[h];
  bf16* yout = static_cast<bf16*>(a.y) + ((int64_t)rt.row0[r] + s_begin) * nh * P + (int64_t)h * P;
#pragma unroll
  for (int pt = 0; pt < PB; ++pt) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int tq = t0 + 4 * g + rr;
      if (tq < len) {
        // the element goes through a scalar first: a bit cast of a vector element itself reads the
        // vector's first element
        const short xe = xa[pt][rr];
        const float xq = static_cast<float>(__builtin_bit_cast(bf16, xe));
        yout[(int64_t)tq * nh * P + 16 * pt + li] = from_f32<bf16>(y[pt][rr] + expf(cum[tq]) * ys[pt][rr] + D * xq);
      }
    }
  }
}

bool scan_y_supported(const Shape& sh, int esz) {
  // bf16 heads of up to 128 dimensions take the matrix-core kernel, which stages B and C only
  if (esz == 2 && sh.P <= 128) return (size_t)2 * sh.N * TB * 2 + 2 * TB * sizeof(float) <= 160 * 1024 - 256;
  return (size_t)TB * (sh.P + 2 * sh.N) * esz + 2 * TB * sizeof(float) <= 160 * 1024 - 256;
}

// Workgroup geometry: an output block of PB16 x NB16 tiles of 16 x 16, the largest divisors of
// P / 16 and N / 16 (N first) that keep both at most 8 and the block within SG_MAX_TILES.
struct SegGeo {
  int pb16, nb16, npb, nnb;
};
static SegGeo seg_geo(const Shape& sh) {
  const int P16 = sh.P / 16, N16 = sh.N / 16;
  int nb16 = 1, pb16 = 1;
  for (int d = 1; d <= SG_MAX_T16; ++d)
    if (N16 % d == 0) nb16 = d;
  for (int d = 1; d <= SG_MAX_T16; ++d)
    if (P16 % d == 0 && d * nb16 <= SG_MAX_TILES) pb16 = d;
  return {pb16, nb16, P16 / pb16, N16 / nb16};
}

int64_t scan_items_per_seg(const Shape& sh) {
  const SegGeo g = seg_geo(sh);
  return (int64_t)sh.nh * g.npb * g.nnb;
}

// LDS of one workgroup: the pre-pass scratch, one weight per token (whole macro-steps) and a
// staged block of H (unpitched rows); afterwards two row-major accumulator blocks (row pitch
// NB + 4).
static size_t scan_acc_block_bytes(const Shape& sh) {
  const SegGeo g = seg_geo(sh);
  return sizeof(float) * (16 * g.pb16) * (16 * g.nb16 + 4);
}
static size_t scan_lds_bytes(const Shape& sh, int esz, int64_t seg_tokens) {
  const int64_t ms = 128 / esz;
  const size_t main_bytes = sizeof(float) * (64 + (seg_tokens + ms - 1) / ms * ms) + scan_acc_block_bytes(sh);
  const size_t red_bytes = 2 * scan_acc_block_bytes(sh);
  return main_bytes > red_bytes ? main_bytes : red_bytes;
}

// Longest segment: its weights fit in LDS next to the staged H, and its blocks span less than
// 2 GiB of the widest time-blocked tensor a caller passes (x and B in one buffer: nh P + G N
// feature rows), so buffer offsets stay 32-bit.
int64_t scan_max_seg_tokens(const Shape& sh, int esz) {
  const int64_t lds_cap = ((int64_t)160 * 1024 - 64 * 4 - (int64_t)scan_acc_block_bytes(sh)) / 4 / TB * TB;
  const int64_t blk_bytes = (int64_t)(sh.dq + sh.gn) * TB * esz;
  int64_t off_cap = (int64_t)0x7fffffff / blk_bytes * TB;
  if (off_cap < TB) off_cap = TB;
  return off_cap < lds_cap ? off_cap : lds_cap;
}

typedef hipError_t (*SegLaunch)(const Shape&, const ScanArgs&, const ReqTable&, hipStream_t);

template <typename T, int PB16, int NB16>
static hipError_t launch_seg_t(const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  const SegGeo g = seg_geo(sh);
  const int n_items = (int)(a.total_segs * scan_items_per_seg(sh));
  const int per_xcd = (n_items + 7) / 8;
  const size_t lds = scan_lds_bytes(sh, sizeof(T), a.seg_tokens);
  static std::once_flag once;
  static hipError_t set_err = hipSuccess;
  std::call_once(once, [] {
    set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_ssd_seg<T, PB16, NB16>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (set_err != hipSuccess) return set_err;
  hipLaunchKernelGGL((k_ssd_seg<T, PB16, NB16>), dim3(8 * per_xcd), dim3(SG_THREADS), lds, s, sh, a, rt, g.npb,
                     g.nnb, n_items, per_xcd);
  return hipGetLastError();
}

// One instantiation per (PB16, NB16) pair within the tile budget; entry (pb16 - 1) * 8 + nb16 - 1.
template <typename T, int I>
constexpr SegLaunch seg_entry() {
  constexpr int pb = I / SG_MAX_T16 + 1, nb = I % SG_MAX_T16 + 1;
  if constexpr (pb * nb <= SG_MAX_TILES)
    return &launch_seg_t<T, pb, nb>;
  else
    return nullptr;
}
template <typename T, size_t... I>
constexpr std::array<SegLaunch, sizeof...(I)> seg_table(std::index_sequence<I...>) {
  return {seg_entry<T, (int)I>()...};
}

template <typename T>
static hipError_t launch_seg(const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  static constexpr std::array<SegLaunch, SG_MAX_T16 * SG_MAX_T16> table =
      seg_table<T>(std::make_index_sequence<SG_MAX_T16 * SG_MAX_T16>());
  const SegGeo g = seg_geo(sh);
  const SegLaunch f = table[(g.pb16 - 1) * SG_MAX_T16 + g.nb16 - 1];
  return f ? f(sh, a, rt, s) : hipErrorInvalidValue;
}

template <typename T, int MAXT>
static hipError_t launch_y_t(const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  size_t lds = (size_t)TB * (sh.P + 2 * sh.N) * sizeof(T) + 2 * TB * sizeof(float);
  // the block's starting state goes to LDS too when it fits (N a multiple of 32 for its swizzle)
  const size_t h0b = (size_t)sh.P * sh.N * sizeof(float);
  const int h0_lds = sh.N % 32 == 0 && lds + h0b <= 160 * 1024 - 256 ? 1 : 0;
  if (h0_lds) lds += h0b;
  static std::once_flag once;
  static hipError_t set_err = hipSuccess;
  std::call_once(once, [] {
    set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_ssd_y<T, MAXT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
  });
  if (set_err != hipSuccess) return set_err;
  hipLaunchKernelGGL((k_ssd_y<T, MAXT>), dim3(a.total_segs * sh.nh), dim3(256), lds, s, sh, a, rt, h0_lds);
  return hipGetLastError();
}

template <int PB>
static hipError_t launch_y_mfma_t(const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  const size_t lds = (size_t)2 * sh.N * TB * 2 + 2 * TB * sizeof(float);
  static std::once_flag once;
  static hipError_t set_err = hipSuccess;
  std::call_once(once, [] {
    set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_ssd_y_mfma<PB>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
  });
  if (set_err != hipSuccess) return set_err;
  hipLaunchKernelGGL(k_ssd_y_mfma<PB>, dim3(a.total_segs * sh.nh), dim3(512), lds, s, sh, a, rt);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_y(const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    // heads of up to 128 dimensions on the bf16 matrix cores
    switch (sh.P / 16) {
      case 1: return launch_y_mfma_t<1>(sh, a, rt, s);
      case 2: return launch_y_mfma_t<2>(sh, a, rt, s);
      case 3: return launch_y_mfma_t<3>(sh, a, rt, s);
      case 4: return launch_y_mfma_t<4>(sh, a, rt, s);
      case 5: return launch_y_mfma_t<5>(sh, a, rt, s);
      case 6: return launch_y_mfma_t<6>(sh, a, rt, s);
      case 7: return launch_y_mfma_t<7>(sh, a, rt, s);
      case 8: return launch_y_mfma_t<8>(sh, a, rt, s);
      default: break;
    }
  }
  return sh.P > 128 ? launch_y_t<T, 16>(sh, a, rt, s) : launch_y_t<T, 8>(sh, a, rt, s);
}

template <int PB>
static hipError_t launch_blk_state_t(const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  const size_t lds = (size_t)(PB + sh.N / 16) * (TB / 32) * 1024 + TB * sizeof(float);
  static std::once_flag once;
  static hipError_t set_err = hipSuccess;
  std::call_once(once, [] {
    set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_ssd_blk_state<PB>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
  });
  if (set_err != hipSuccess) return set_err;
  hipLaunchKernelGGL(k_ssd_blk_state<PB>, dim3(a.total_segs * sh.nh), dim3(256), lds, s, sh, a, rt);
  return hipGetLastError();
}

// The states of y-mode blocks: bf16 heads of up to 128 dimensions on the matrix-core block kernel,
// the rest on the segment kernel (segments of one block).
static hipError_t launch_y_states(int dtype, const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  if (dtype == HYF_BF16) {
    switch (sh.P / 16) {
      case 1: return launch_blk_state_t<1>(sh, a, rt, s);
      case 2: return launch_blk_state_t<2>(sh, a, rt, s);
      case 3: return launch_blk_state_t<3>(sh, a, rt, s);
      case 4: return launch_blk_state_t<4>(sh, a, rt, s);
      case 5: return launch_blk_state_t<5>(sh, a, rt, s);
      case 6: return launch_blk_state_t<6>(sh, a, rt, s);
      case 7: return launch_blk_state_t<7>(sh, a, rt, s);
      case 8: return launch_blk_state_t<8>(sh, a, rt, s);
      default: return launch_seg<bf16>(sh, a, rt, s);
    }
  }
  return launch_seg<float>(sh, a, rt, s);
}

hipError_t launch_ssd_state(int dtype, const Shape& sh, const ScanArgs& a, const ReqTable& rt,
                            int32_t max_segs_per_req, hipStream_t s) {
  if (a.total_segs <= 0) return hipSuccess;
  hipError_t e = a.y_mode ? launch_y_states(dtype, sh, a, rt, s)
                          : dtype == HYF_BF16 ? launch_seg<bf16>(sh, a, rt, s) : launch_seg<float>(sh, a, rt, s);
  if (e != hipSuccess) return e;
  const int64_t PN = (int64_t)sh.P * sh.N;
  dim3 grid((unsigned)rt.n_req * sh.nh, (unsigned)((PN / 4 + 255) / 256));
  if (!a.y_mode) {
    if (max_segs_per_req <= 1) return hipSuccess;
    hipLaunchKernelGGL(k_ssd_combine, grid, dim3(256), 0, s, sh, a, rt);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_ssd_prefix, grid, dim3(256), 0, s, sh, a, rt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return dtype == HYF_BF16 ? launch_y<bf16>(sh, a, rt, s) : launch_y<float>(sh, a, rt, s);
}

}  // namespace hyf
