// Kernels of one draft/commit round (k_round, see below) and the ring/state helpers of a prefill
// commit (k_ring_append, k_bump_counts, k_reset_states, k_zero).
#include <mutex>

#include "hyf_launch.h"

namespace hyf {

constexpr int RB = HYF_BLOCK;   // block rows
constexpr int RMAXC = 16;       // largest per-request commit a round kernel folds in
constexpr int KS_MIN = 64;      // fewest keys per attention split (the workspace is sized for it)
constexpr int WIDE_PASSES = 16; // most row passes of one commit / readout tile (wide layout)
constexpr int MID_PASSES = 2;   // most row passes of a tile in the narrow layout (3 spills at 80 VGPRs)
constexpr int RT = 256;         // threads per round workgroup

__device__ __forceinline__ int64_t* count_ptr(char* pool, const Shape& sh, int slot) {
  return reinterpret_cast<int64_t*>(pool + (int64_t)slot * sh.st_bytes);
}
__device__ __forceinline__ float* h_ptr(char* pool, const Shape& sh, int slot, int h) {
  return reinterpret_cast<float*>(pool + (int64_t)slot * sh.st_bytes + sh.st_h) + (int64_t)h * sh.P * sh.N;
}
template <typename T>
__device__ __forceinline__ T* ring_ptr(char* pool, const Shape& sh, int slot, uint64_t off, int h) {
  return reinterpret_cast<T*>(pool + (int64_t)slot * sh.st_bytes + off) + (int64_t)h * sh.W * sh.P;
}

// Committed rows of request r in this round: from the host table, or from device memory (clamped to
// 0..RB) when the caller passes the counts on the device.
__device__ __forceinline__ int commit_rows(const RoundArgs& a, const ReqTable& rt, int r) {
  if (a.dev_rows) return min(max(a.dev_rows[r], 0), RB);
  return rt.row0[r + 1] - rt.row0[r];
}

// ---------------------------------------------------------------------------------------------
// One round, one launch.  Workgroup roles per (request r, head h), in block-index order:
//   tiles  [0, n_tiles):   rows p0 .. p0 + tile_rows of H: fold the round's committed rows in (one
//                          read-modify-write), memory readout of the block rows from the updated
//                          rows, and (tile 0) the ring append of the committed (k, v);
//   splits [n_tiles, +n_split): attention of the 8 block rows over ks ring slots (the last split:
//                          over the block rows themselves), written as (max, sum, output) partials.
// The layout (ks, tile_rows) is chosen per launch (round_layout).
// A split sees the ring as it is after this round's append without waiting for it: a slot that
// the append overwrites is read from the projection instead (rounded to the storage dtype, as the
// ring stores it).  The last workgroup of (r, h) to finish (a counter) merges the splits, adds the
// readout and writes the output projection's input; the last head of a request advances the
// request's committed count.  The counters are cleared by the round's input projection.
//
// Memory ordering of the hand-over: every partial result a workgroup leaves for the merge (the
// attention partials, the (max, sum) pairs, the readout) is written with device-scope stores that
// bypass the non-coherent per-XCD caches (st_dev), and the writer waits for all of its stores to be
// acknowledged (vm_wait<0>) before the barrier after which one thread increments the (r, h) counter.
// The workgroup that sees the counter reach its final value therefore runs after every store of the
// other workgroups of (r, h) has reached the device-coherent level, and it reads the partials with
// device-coherent loads (sc1), so it cannot see stale copies.  The atomic itself needs no fence: the
// order comes from the completed stores before it, not from the atomic's own ordering.

// Staging: a job copies n chunks (16 or 4 bytes) from global memory, chunk i from src(i) to
// dst + i chunks in LDS, with direct global -> LDS loads: no registers and no wait between
// loads, so every job of a workgroup is one memory round trip.  A wave issues chunks
// [64 k, 64 k + 64) for k = wave, wave + 4, ...; LDS regions are sized in whole 1 KiB (16-byte
// jobs) or 256-byte (4-byte jobs) units so a wave's instruction stays inside its region.
template <typename F>
__device__ __forceinline__ void stage16(int n, void* dst, F src) {
  lds_stage16<RT>(n, dst, src);
}
template <typename F>
__device__ __forceinline__ void stage4(int n, void* dst, F src) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int base = wave * 64; base < n; base += RT)
    if (base + lane < n) lds_dma4(src(base + lane), static_cast<char*>(dst) + 4 * base);
}
__host__ __device__ constexpr int up1k(int bytes) { return (bytes + 1023) / 1024 * 1024; }

// count mod W for 0 <= count < 2^52 (one double division instead of a 64-bit integer division: the
// rounded quotient is within one of the true one, and one step corrects the remainder).
__device__ __forceinline__ int mod_w(int64_t count, int W) {
  const int64_t q = (int64_t)((double)count / (double)W);
  int64_t r = count - q * W;
  if (r < 0) r += W;
  else if (r >= W) r -= W;
  return (int)r;
}

// Results another workgroup of the same launch merges are stored device-coherent (written through
// to the level all XCDs share) and read the same way, so the hand-over needs no L2 write-back or
// invalidation: the writer waits for its stores to complete before it counts itself in.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr int AUX_DEV = 16;  // cache policy of a device-coherent load (sc1)
template <typename F>
__device__ __forceinline__ void stage16_dev(int n, void* dst, F src) {
  lds_stage16<RT, AUX_DEV>(n, dst, src);
}

// Tile LDS (bytes): B of the committed rows [RMAXC][N] f32 | C of the block rows [RB][N] f32 |
// x (= v) of the committed rows [RMAXC][tile_rows] f32 | v of the block rows [RB][tile_rows] f32 |
// weights [RMAXC + 4] (gated delta rule: retention gates) | write gates [RMAXC] | inverse key norms
// [RMAXC] | inverse query norms [RB] | readout partials [RB][RT].
//
// A tile's threads hold tpr = N / 4 threads per row of H (4 columns each), rows_wg = RT / tpr rows
// at a time; a tile of tile_rows rows takes tile_rows / rows_wg passes, every pass's row of H in
// registers, all of them loaded before any arithmetic.  Several passes need tpr a power of two (the
// row reductions are lane shuffles); otherwise a tile is one pass.
//
// Gated delta-rule memory (sh.gdn): the committed rows are folded one at a time, each row of H
// (tpr threads) forming H_p . k with a reduction over its threads, then
// H_p <- alpha (H_p - beta (H_p . k) k) + beta x_p k, k the unit-normalized B row; the readout
// uses the unit-normalized C rows.
template <typename T, int TMAXG>
__device__ __forceinline__ void round_tile(const Shape& sh, const RoundArgs& a, const ReqTable& rt, int r, int h,
                                           int tile, char* smem) {
  const int nh = sh.nh, P = sh.P, N = sh.N;
  const int tpr = N / 4;           // threads per H row (4 columns each)
  const int rows_wg = RT / tpr;    // H rows per pass
  const int trows = a.tile_rows;   // H rows per tile: a multiple of rows_wg, at most TMAXG passes (host-checked)
  const int npass = trows / rows_wg;
  const int t = threadIdx.x;
  const Div& dtpr = a.d_tpr;
  const Div& dtr = a.d_tr;
  const int prow = dtpr.q(t), c4 = t - prow * tpr;
  const int p0 = tile * trows;
  const bool lane_ok = prow < rows_wg;
  const int slot = rt.slot[r];
  const int grp = h / (nh / sh.G);
  const int nrows = a.do_commit ? commit_rows(a, rt, r) : 0;
  const int64_t crow0 = a.dev_rows ? (int64_t)RB * r : rt.row0[r];
  const int64_t brow0 = a.blk_row0 + (int64_t)r * RB;
  const int64_t ld = a.ld;
  float* Bl = reinterpret_cast<float*>(smem);
  float* Cl = reinterpret_cast<float*>(smem + up1k(RMAXC * N * 4));
  float* xv = reinterpret_cast<float*>(reinterpret_cast<char*>(Cl) + up1k(RB * N * 4));
  float* vb = reinterpret_cast<float*>(reinterpret_cast<char*>(xv) + up1k(RMAXC * trows * 4));
  float* wl = reinterpret_cast<float*>(reinterpret_cast<char*>(vb) + up1k(RB * trows * 4));
  float* ga = wl + RMAXC + 4;  // write gates (gated delta rule)
  float* ik = ga + RMAXC;      // inverse key norms
  float* iq = ik + RMAXC;      // inverse query norms
  float* red = iq + RB;

  // every load first (one round trip), then the arithmetic
  float* Hh = h_ptr(a.state_pool, sh, slot, h);
  f32x4 hv[TMAXG];
#pragma unroll
  for (int i = 0; i < TMAXG; ++i) {
    hv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int p = p0 + prow + i * rows_wg;
    if (i < npass && lane_ok && p < P) hv[i] = *reinterpret_cast<const f32x4*>(Hh + (int64_t)p * N + 4 * c4);
  }
  const float raw = t < nrows ? a.proj[(crow0 + t) * ld + sh.off_dt + h] : 0.f;
  const float rawb = sh.gdn && t < nrows ? a.proj[(crow0 + t) * ld + sh.off_beta + h] : 0.f;
  // column of tile row i (rows past the head's last row read its last row; their values go unused)
  auto tcol = [&](int i) { return p0 + i < P ? p0 + i : P - 1; };
  // row q of a staging job sits q ld floats past the job's first row (ld (RMAXC + RB) < 2^31 / 4)
  const int ldi = (int)ld;
  const float* cb = a.proj + crow0 * ld + sh.off_b + grp * N;
  const float* cv = a.proj + crow0 * ld + sh.off_v + h * P;
  stage16(nrows * tpr, Bl, [&](int i) { const int q = dtpr.q(i); return cb + (uint32_t)(q * ldi + 4 * (i - q * tpr)); });
  stage4(nrows * trows, xv, [&](int i) { const int q = dtr.q(i); return cv + (uint32_t)(q * ldi + tcol(i - q * trows)); });
  if (a.do_draft) {
    const float* bc = a.proj + brow0 * ld + sh.off_c + grp * N;
    const float* bv = a.proj + brow0 * ld + sh.off_v + h * P;
    stage16(RB * tpr, Cl, [&](int i) { const int q = dtpr.q(i); return bc + (uint32_t)(q * ldi + 4 * (i - q * tpr)); });
    stage4(RB * trows, vb, [&](int i) { const int q = dtr.q(i); return bv + (uint32_t)(q * ldi + tcol(i - q * trows)); });
  }
  if (sh.gdn) {
    if (t < nrows) {
      wl[t] = 1.f / (1.f + __expf(-(raw + a.dt_bias[h])));  // retention gate (its bias in dt_bias)
      ga[t] = 1.f / (1.f + __expf(-(rawb + a.a_log[h])));   // write gate (its bias in a_log)
    }
  } else if (t < 64) {
    // weights relative to the last committed row: w_t = dt_t exp(sum_{tau > t} dt_tau A), and
    // the decay exp(sum_t dt_t A) of the old state; lane t < nrows holds row t
    const float A = -expf(a.a_log[h]);
    const float dt = t < nrows ? softplus_f(raw + a.dt_bias[h]) : 0.f;
    const float ell = dt * A;
    float inc = ell;  // sum over lanes t .. RMAXC - 1
#pragma unroll
    for (int o = 1; o < RMAXC; o <<= 1) {
      const float v = __shfl_down(inc, o, 64);
      if (t + o < RMAXC) inc += v;
    }
    if (t < nrows) wl[t] = dt * expf(inc - ell);
    if (t == 0) wl[RMAXC] = expf(inc);
  }
  vm_wait<0>();
  __syncthreads();

  const bool pow2 = (tpr & (tpr - 1)) == 0;  // the tpr threads of a row are consecutive lanes of one wave
  if (sh.gdn) {
    // inverse norms of the committed rows' keys and the block rows' queries, one row per wave at a time
    const int lane = t & 63, wave = t >> 6;
    for (int j = wave; j < nrows + (a.do_draft ? RB : 0); j += RT / 64) {
      const float* row = j < nrows ? Bl + j * N : Cl + (j - nrows) * N;
      float ss = 0.f;
      for (int n = lane; n < N; n += 64) ss += row[n] * row[n];
      ss = wave_sum(ss);
      if (lane == 0) {
        if (j < nrows) ik[j] = rsqrtf(ss + 1e-6f);
        else iq[j - nrows] = rsqrtf(ss + 1e-6f);
      }
    }
    __syncthreads();
    if (nrows > 0) {
      for (int tt = 0; tt < nrows; ++tt) {
        const f32x4 k = *reinterpret_cast<const f32x4*>(Bl + tt * N + 4 * c4) * ik[tt];
        const float be = ga[tt];
        if (pow2) {
#pragma unroll
          for (int i = 0; i < TMAXG; ++i) {
            if (i < npass) {
              float d = hv[i][0] * k[0] + hv[i][1] * k[1] + hv[i][2] * k[2] + hv[i][3] * k[3];
              for (int o = tpr / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
              const int pr = prow + i * rows_wg;
              const float xw = lane_ok && p0 + pr < P ? be * xv[tt * trows + pr] : 0.f;
              hv[i] = wl[tt] * (hv[i] - (be * d) * k) + xw * k;
            }
          }
        } else {
          // one pass (the host keeps tile_rows = rows_wg here)
          float d = hv[0][0] * k[0] + hv[0][1] * k[1] + hv[0][2] * k[2] + hv[0][3] * k[3];
          red[t] = d;
          __syncthreads();
          d = 0.f;
          if (lane_ok)
            for (int c = 0; c < tpr; ++c) d += red[prow * tpr + c];
          __syncthreads();
          const float xw = lane_ok && p0 + prow < P ? be * xv[tt * trows + prow] : 0.f;
          hv[0] = wl[tt] * (hv[0] - (be * d) * k) + xw * k;
        }
      }
    }
  } else if (nrows > 0 && !sh.lastw) {
    const float dec = wl[RMAXC];
#pragma unroll
    for (int i = 0; i < TMAXG; ++i)
      if (i < npass) hv[i] *= dec;
    for (int tt = 0; tt < nrows; ++tt) {
      const f32x4 b = *reinterpret_cast<const f32x4*>(Bl + tt * N + 4 * c4);
      const float w = wl[tt];
#pragma unroll
      for (int i = 0; i < TMAXG; ++i) {
        if (i < npass) {
          const int pr = prow + i * rows_wg;
          const float xw = lane_ok && p0 + pr < P ? xv[tt * trows + pr] * w : 0.f;
          hv[i] += xw * b;
        }
      }
    }
  }
  if (nrows > 0 && !sh.lastw) {
#pragma unroll
    for (int i = 0; i < TMAXG; ++i) {
      const int p = p0 + prow + i * rows_wg;
      if (i < npass && lane_ok && p < P) *reinterpret_cast<f32x4*>(Hh + (int64_t)p * N + 4 * c4) = hv[i];
    }
  }

  if (a.do_draft) {
    const float D = a.d_skip[h];
    if (pow2) {
#pragma unroll
      for (int i = 0; i < TMAXG; ++i) {
        if (i >= npass) continue;
        float sum[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const f32x4 c = *reinterpret_cast<const f32x4*>(Cl + j * N + 4 * c4);
          sum[j] = hv[i][0] * c[0] + hv[i][1] * c[1] + hv[i][2] * c[2] + hv[i][3] * c[3];
        }
        // the tpr threads of a row are consecutive lanes of one wave.  With tpr >= 8 the 8 sums are
        // reduced by halving: at offsets tpr/2, tpr/4, tpr/8 a lane keeps half of its sums (the upper
        // half if its offset bit is set) and adds its partner's copies of them, so after three steps
        // lane c4 holds one sum, of block row j = (c4 / (tpr / 8)) mod 8, and the offsets below
        // tpr/8 finish it (9 shuffles for tpr = 32 instead of 40).
        const int pr = prow + i * rows_wg;
        if (tpr >= 8) {
          {
            const int o = tpr >> 1;
            const bool hi = (c4 & o) != 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float send = hi ? sum[k] : sum[k + 4], keep = hi ? sum[k + 4] : sum[k];
              sum[k] = keep + __shfl_xor(send, o, 64);
            }
          }
          {
            const int o = tpr >> 2;
            const bool hi = (c4 & o) != 0;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              const float send = hi ? sum[k] : sum[k + 2], keep = hi ? sum[k + 2] : sum[k];
              sum[k] = keep + __shfl_xor(send, o, 64);
            }
          }
          {
            const int o = tpr >> 3;
            const bool hi = (c4 & o) != 0;
            const float send = hi ? sum[0] : sum[1], keep = hi ? sum[1] : sum[0];
            sum[0] = keep + __shfl_xor(send, o, 64);
          }
          for (int o = tpr >> 4; o >= 1; o >>= 1) sum[0] += __shfl_xor(sum[0], o, 64);
          const int sub = tpr >> 3;
          const int j = (c4 / sub) & 7;
          if (lane_ok && c4 % sub == 0 && p0 + pr < P)
            st_dev(a.mem + (((int64_t)r * RB + j) * nh + h) * P + p0 + pr,
                   sum[0] * (sh.gdn ? iq[j] : 1.f) + D * vb[j * trows + pr]);
        } else {
          for (int o = tpr / 2; o >= 1; o >>= 1)
#pragma unroll
            for (int j = 0; j < RB; ++j) sum[j] += __shfl_xor(sum[j], o, 64);
          if (lane_ok && c4 == 0 && p0 + pr < P)
#pragma unroll
            for (int j = 0; j < RB; ++j)
              st_dev(a.mem + (((int64_t)r * RB + j) * nh + h) * P + p0 + pr,
                     sum[j] * (sh.gdn ? iq[j] : 1.f) + D * vb[j * trows + pr]);
        }
      }
    } else {
      float sum[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(Cl + j * N + 4 * c4);
        sum[j] = lane_ok ? hv[0][0] * c[0] + hv[0][1] * c[1] + hv[0][2] * c[2] + hv[0][3] * c[3] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < RB; ++j) red[j * RT + t] = sum[j];
      __syncthreads();
      for (int idx = t; idx < RB * rows_wg; idx += RT) {
        const int j = idx / rows_wg, pr = idx % rows_wg;
        const int pp = p0 + pr;
        if (pp >= P) continue;
        float acc = 0.f;
        for (int c = 0; c < tpr; ++c) acc += red[j * RT + pr * tpr + c];
        st_dev(a.mem + (((int64_t)r * RB + j) * nh + h) * P + pp,
               acc * (sh.gdn ? iq[j] : 1.f) + D * vb[j * trows + pr]);
      }
    }
  }

  // ring append of this round's rows (tile 0 of each head): the last min(n, W) rows
  if (tile == 0 && nrows > 0) {
    const int64_t count = *count_ptr(a.state_pool, sh, slot);
    const int W = sh.W;
    const int first = nrows > W ? nrows - W : 0;
    T* K = ring_ptr<T>(a.state_pool, sh, slot, sh.st_k, h);
    T* V = ring_ptr<T>(a.state_pool, sh, slot, sh.st_v, h);
    const int cw = mod_w(count, W);
    for (int tt = first; tt < nrows; ++tt) {
      int s = cw + tt;
      while (s >= W) s -= W;  // uniform
      for (int pp = t; pp < P; pp += RT) {
        K[s * P + pp] = from_f32<T>(a.proj[(crow0 + tt) * ld + sh.off_k + h * P + pp]);
        V[s * P + pp] = from_f32<T>(a.proj[(crow0 + tt) * ld + sh.off_v + h * P + pp]);
      }
      if (sh.lastw) {
        // the B row (one head per group writes it) and the raw step of the row, for the rescan
        char* blob = a.state_pool + (int64_t)slot * sh.st_bytes;
        if (t == 0) reinterpret_cast<float*>(blob + sh.st_dt)[(int64_t)h * W + s] = a.proj[(crow0 + tt) * ld + sh.off_dt + h];
        if (h % (nh / sh.G) == 0)
          for (int n = t; n < N; n += RT)
            reinterpret_cast<T*>(blob + sh.st_b)[s * sh.gn + grp * N + n] =
                from_f32<T>(a.proj[(crow0 + tt) * ld + sh.off_b + grp * N + n]);
      }
    }
  }
}

// Eight consecutive elements (16-byte aligned) as fp32, and two as fp32 (4-byte aligned bf16,
// 8-byte aligned fp32).
__device__ __forceinline__ void ld8f(const float* p, float* o) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = a[i];
    o[4 + i] = b[i];
  }
}
__device__ __forceinline__ void ld8f(const bf16* p, float* o) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = static_cast<float>(v[i]);
}
__device__ __forceinline__ void ld2f(const float* p, float& x, float& y) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  const f32x2 v = *reinterpret_cast<const f32x2*>(p);
  x = v[0];
  y = v[1];
}
__device__ __forceinline__ void ld2f(const bf16* p, float& x, float& y) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 v = *reinterpret_cast<const bf16x2*>(p);
  x = static_cast<float>(v[0]);
  y = static_cast<float>(v[1]);
}

// Attention of the 8 block rows over nk keys (at most ks) of one split, on the vector ALUs: wave w
// owns queries 2w and 2w + 1 (fp32, qs [RB][P]); lane l scores keys l, l + 64, ... against both
// (dot products over P with the key row read from LDS, 8 elements at a time; the query rows are
// read by every lane at once, a broadcast), so the softmax of a query is a reduction inside one
// wave.  The probabilities go to the wave's two rows of pl ([RB][ks + 4]); then lane l forms
// output columns 2l, 2l + 1 (and 2l + 128, 2l + 129 when P > 128) of both queries, key by key.
// Keys at or past nk are masked (their rows may hold anything; they are never read).
template <typename KT>
__device__ __forceinline__ void attn_split(const Shape& sh, int nk, int ks, bool blk, const float* qs, const KT* K,
                                           const KT* V, float* pl, float* red, float* op, float* ml) {
  (void)red;
  const int P = sh.P, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int q0 = 2 * wave, q1 = q0 + 1;
  const float scale = rsqrtf((float)P);
  const int pls = ks + 4;
  float m0 = -INFINITY, m1 = -INFINITY;
  // ---- scores of this lane's keys
  for (int key = lane; key < ks; key += 64) {
    float s0 = -INFINITY, s1 = -INFINITY;
    if (key < nk) {
      const KT* kr = K + key * P;
      float a0 = 0.f, a1 = 0.f;
#pragma unroll 2
      for (int p0 = 0; p0 < P; p0 += 8) {
        float kv[8], qa[8], qb[8];
        ld8f(kr + p0, kv);
        ld8f(qs + q0 * P + p0, qa);
        ld8f(qs + q1 * P + p0, qb);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a0 = fmaf(kv[i], qa[i], a0);
          a1 = fmaf(kv[i], qb[i], a1);
        }
      }
      s0 = a0 * scale;
      s1 = a1 * scale;
      if (blk && !sh.cross) {  // block keys: each row sees only itself
        if (key != q0) s0 = -INFINITY;
        if (key != q1) s1 = -INFINITY;
      }
    }
    pl[q0 * pls + key] = s0;
    pl[q1 * pls + key] = s1;
    m0 = fmaxf(m0, s0);
    m1 = fmaxf(m1, s1);
  }
  m0 = wave_max64(m0);
  m1 = wave_max64(m1);
  float l0 = 0.f, l1 = 0.f;
  for (int key = lane; key < ks; key += 64) {
    const float e0 = pl[q0 * pls + key], e1 = pl[q1 * pls + key];
    const float p0 = e0 == -INFINITY ? 0.f : __expf(e0 - m0);
    const float p1 = e1 == -INFINITY ? 0.f : __expf(e1 - m1);
    pl[q0 * pls + key] = p0;
    pl[q1 * pls + key] = p1;
    l0 += p0;
    l1 += p1;
  }
  l0 = wave_sum64(l0);
  l1 = wave_sum64(l1);
  if (lane == 0) {
    st_dev(ml + 2 * q0, m0);
    st_dev(ml + 2 * q0 + 1, l0);
    st_dev(ml + 2 * q1, m1);
    st_dev(ml + 2 * q1 + 1, l1);
  }
  // the wave's probability rows are read by all of its lanes below
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // ---- O[q][p] = sum_key p[q][key] V[key][p], four keys per step
  const float* pr0 = pl + q0 * pls;
  const float* pr1 = pl + q1 * pls;
  for (int c = 2 * lane; c < P; c += 128) {
    float o00 = 0.f, o01 = 0.f, o10 = 0.f, o11 = 0.f;
    const KT* vc = V + c;
    int key = 0;
    for (; key + 4 <= nk; key += 4) {
      const f32x4 pa = *reinterpret_cast<const f32x4*>(pr0 + key);
      const f32x4 pb = *reinterpret_cast<const f32x4*>(pr1 + key);
      float vx[4], vy[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) ld2f(vc + (key + u) * P, vx[u], vy[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        o00 = fmaf(pa[u], vx[u], o00);
        o01 = fmaf(pa[u], vy[u], o01);
        o10 = fmaf(pb[u], vx[u], o10);
        o11 = fmaf(pb[u], vy[u], o11);
      }
    }
    for (; key < nk; ++key) {
      float vx, vy;
      ld2f(vc + key * P, vx, vy);
      o00 = fmaf(pr0[key], vx, o00);
      o01 = fmaf(pr0[key], vy, o01);
      o10 = fmaf(pr1[key], vx, o10);
      o11 = fmaf(pr1[key], vy, o11);
    }
    st_dev(op + q0 * P + c, o00);
    st_dev(op + q0 * P + c + 1, o01);
    st_dev(op + q1 * P + c, o10);
    st_dev(op + q1 * P + c + 1, o11);
  }
}

// Attention of the 8 block rows over nk keys (at most ks, ks a multiple of 16, at most 128) of a
// bf16 ring split, on bf16 matrix cores (16x16x16, fp32 accumulation), near fp32 accuracy: the
// fp32 queries and probabilities enter as two bf16 terms each (hi = bf16(x), lo = bf16(x - hi),
// together within 2^-16 of x), the ring's keys and values are bf16 already, and every product of
// bf16 operands is exact in fp32.
//   scores:  wave w takes key tiles w, w + 4 (16 keys each): S^T = K Q^T, A = 16 keys x 16 dims
//            of K (LDS), B = 16 dims x 16 queries (rows 8..15 repeat rows 0..7 and go unused);
//            lane l ends with keys 16 kt + 4 (l / 16) + r (r = 0..3) of query l % 16 in registers.
//   softmax: the split's maximum per query over the four waves (LDS), then p = exp(s - max).
//   values:  those registers are already the A operand of O = P V (query l % 16, keys
//            4 (l / 16) + r of the tile), B = V[keys][16 dims], four 2-byte LDS reads per lane;
//            the waves' products (same maximum) are summed through LDS in wave order.
// Ring rows past nk may hold anything: their scores are replaced (not multiplied) by -inf, and
// their value rows are zeroed first, since a zero probability times a NaN would not be zero.
typedef __attribute__((ext_vector_type(4))) short s16x4;
__device__ __forceinline__ short bf16_bits(float v) { return __builtin_bit_cast(short, static_cast<bf16>(v)); }
__device__ __forceinline__ float bf16_val(short b) { return static_cast<float>(__builtin_bit_cast(bf16, b)); }

__device__ __forceinline__ void attn_split_mfma(const Shape& sh, int nk, int ks, float* qs, const bf16* K, bf16* V,
                                                float* red, float* op, float* ml) {
  const int P = sh.P, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int li = lane & 15, g = lane >> 4;
  const float scale = rsqrtf((float)P);
  const int nkt = ks / 16, npc = P / 16;
  // ---- queries -> (hi, lo) bf16 pairs in place: qh [RB][P] then ql [RB][P] over the fp32 rows
  constexpr int QE = RB * 256 / RT;  // elements per thread (P <= 256)
  float qv[QE];
#pragma unroll
  for (int e = 0; e < QE; ++e) qv[e] = t + e * RT < RB * P ? qs[t + e * RT] : 0.f;
  // value rows past nk: zero (16-byte stores)
  if (nk < ks) {
    uint4* vz = reinterpret_cast<uint4*>(V + (int64_t)nk * P);
    const int n16 = (ks - nk) * P / 8;
    for (int i = t; i < n16; i += RT) vz[i] = uint4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  short* qh = reinterpret_cast<short*>(qs);
  short* ql = qh + RB * P;
#pragma unroll
  for (int e = 0; e < QE; ++e) {
    const int i = t + e * RT;
    if (i < RB * P) {
      const short hb = bf16_bits(qv[e]);
      qh[i] = hb;
      ql[i] = bf16_bits(qv[e] - bf16_val(hb));
    }
  }
  __syncthreads();

  // ---- scores of this wave's key tiles
  const short* kb = reinterpret_cast<const short*>(K);
  const int qrow = (li & 7) * P;
  f32x4 s[2];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kt = wave + 4 * j;
    s[j] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (kt < nkt && 16 * kt < nk) {  // uniform
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      const short* kr = kb + (16 * kt + li) * P + 4 * g;
      for (int c = 0; c < npc; ++c) {
        const s16x4 a = *reinterpret_cast<const s16x4*>(kr + 16 * c);
        const s16x4 bh = *reinterpret_cast<const s16x4*>(qh + qrow + 16 * c + 4 * g);
        const s16x4 bl = *reinterpret_cast<const s16x4*>(ql + qrow + 16 * c + 4 * g);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bl, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[j][r] = 16 * kt + 4 * g + r < nk ? acc[r] * scale : -INFINITY;
        mx = fmaxf(mx, s[j][r]);
      }
    }
  }
  // ---- softmax over the split: maximum over the lanes of query li, then over the waves
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (g == 0) red[wave * 16 + li] = mx;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[li], red[16 + li]), fmaxf(red[32 + li], red[48 + li]));
  float lsum = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[j][r] = s[j][r] == -INFINITY ? 0.f : __expf(s[j][r] - m);
      lsum += s[j][r];
    }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (g == 0) red[64 + wave * 16 + li] = lsum;
  // probabilities as (hi, lo) A operands
  s16x4 ph[2], pl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const short hb = bf16_bits(s[j][r]);
      ph[j][r] = hb;
      pl[j][r] = bf16_bits(s[j][r] - bf16_val(hb));
    }

  // ---- O = P V in groups of up to PG dimension tiles; the waves' sums meet in the K region
  float* ob = reinterpret_cast<float*>(const_cast<bf16*>(K));  // [4][RB][16 PG]
  const short* vb = reinterpret_cast<const short*>(V);
  constexpr int PG = 4;  // 16 accumulator registers: the kernel keeps six workgroups per CU
  for (int c0 = 0; c0 < npc; c0 += PG) {
    const int nc = npc - c0 < PG ? npc - c0 : PG;
    f32x4 o[PG];
#pragma unroll
    for (int c = 0; c < PG; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kt = wave + 4 * j;
      if (kt < nkt && 16 * kt < nk) {  // uniform
        const short* vr = vb + (16 * kt + 4 * g) * P + 16 * c0 + li;
#pragma unroll
        for (int c = 0; c < PG; ++c) {
          if (c < nc) {
            s16x4 b;
#pragma unroll
            for (int r = 0; r < 4; ++r) b[r] = vr[r * P + 16 * c];
            o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph[j], b, o[c], 0, 0, 0);
            o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl[j], b, o[c], 0, 0, 0);
          }
        }
      }
    }
    if (c0 > 0) __syncthreads();  // the previous group's sums are read
    // lane l holds O[4 g + r][16 (c0 + c) + li]; rows 0..7 are the queries (g < 2)
    const int gw = 16 * nc;
    if (g < 2) {
#pragma unroll
      for (int c = 0; c < PG; ++c)
        if (c < nc)
#pragma unroll
          for (int r = 0; r < 4; ++r) ob[(wave * RB + 4 * g + r) * gw + 16 * c + li] = o[c][r];
    }
    __syncthreads();
    // wave w sums dimension tile c = w of the group, in the same lane layout
    if (g < 2) {
      {
        const int c = wave;
        if (c < nc) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int o0 = (4 * g + r) * gw + 16 * c + li, wst = RB * gw;
            st_dev(op + (4 * g + r) * P + 16 * (c0 + c) + li, ob[o0] + ob[wst + o0] + ob[2 * wst + o0] + ob[3 * wst + o0]);
          }
        }
      }
    }
  }
  if (t < RB) {
    const float mq = fmaxf(fmaxf(red[t], red[16 + t]), fmaxf(red[32 + t], red[48 + t]));
    st_dev(ml + 2 * t, mq);
    st_dev(ml + 2 * t + 1, red[64 + t] + red[80 + t] + red[96 + t] + red[112 + t]);
  }
}

// Attention LDS (bytes): ring K, V of the split [ks][P] storage dtype (the block split: the block
// rows' k, v [RB][P] f32 in the same places) | q [RB][P] f32 | probabilities [RB][ks + 4] |
// scratch [128].
template <typename T>
__device__ __forceinline__ void round_attn(const Shape& sh, const RoundArgs& a, const ReqTable& rt, int r, int h,
                                           int sp, char* smem) {
  constexpr int VN = Vec16<T>::n;
  constexpr int FIX = (RB * 256 + RT - 1) / RT;  // committed-row elements per thread (P <= 256)
  const int nh = sh.nh, P = sh.P, W = sh.W, ks = a.ks;
  const int kvb = up1k(ks * P * (int)sizeof(T)) > up1k(RB * P * 4) ? up1k(ks * P * (int)sizeof(T)) : up1k(RB * P * 4);
  T* kst = reinterpret_cast<T*>(smem);
  T* vst = reinterpret_cast<T*>(smem + kvb);
  float* qs = reinterpret_cast<float*>(smem + 2 * kvb);
  float* pl = reinterpret_cast<float*>(reinterpret_cast<char*>(qs) + up1k(RB * P * 4));
  float* red = pl + RB * (ks + 4);
  const int slot = rt.slot[r];
  const int t = threadIdx.x;
  const int64_t ld = a.ld;
  const int64_t brow0 = a.blk_row0 + (int64_t)r * RB;
  const bool blk = sp == a.n_split - 1;
  const int nrows = a.do_commit ? commit_rows(a, rt, r) : 0;
  const int64_t crow0 = a.dev_rows ? (int64_t)RB * r : rt.row0[r];
  const int k0 = sp * ks;
  const int P4 = P / 4;

  // Every load is independent of the committed count, so all go out together: q, the split's ring
  // slots (always inside the ring) or the block rows' k, v, and (into registers) the k, v of the
  // round's last committed rows, which replace the slots this round's append overwrites.
  const Div& dP4 = a.d_p4;
  const Div& dP = a.d_p;
  const int ldi = (int)ld;  // rows of one job lie q ld floats apart (ld (RMAXC + RB) < 2^31 / 4)
  const float* bq = a.proj + brow0 * ld + h * P;
  stage16(RB * P4, qs, [&](int i) { const int q = dP4.q(i); return bq + (uint32_t)(sh.off_q + q * ldi + 4 * (i - q * P4)); });
  const int m = nrows < W ? nrows : W;  // committed rows that land in the ring
  // the committed rows' k, v in registers: thread t holds column pc of rows jr, jr + rpp, ...
  const int rpp = dP.q(RT);  // rows per pass (P <= 256)
  const int jr = dP.q(t), pc = t - jr * P;
  float fk[FIX], fv[FIX];
  if (blk) {
    float* bk = reinterpret_cast<float*>(kst);
    float* bv = reinterpret_cast<float*>(vst);
    stage16(RB * P4, bk, [&](int i) { const int q = dP4.q(i); return bq + (uint32_t)(sh.off_k + q * ldi + 4 * (i - q * P4)); });
    stage16(RB * P4, bv, [&](int i) { const int q = dP4.q(i); return bq + (uint32_t)(sh.off_v + q * ldi + 4 * (i - q * P4)); });
  } else {
    const int nslots = W - k0 < ks ? W - k0 : ks;
    const T* K = ring_ptr<T>(a.state_pool, sh, slot, sh.st_k, h) + (int64_t)k0 * P;
    const T* V = ring_ptr<T>(a.state_pool, sh, slot, sh.st_v, h) + (int64_t)k0 * P;
    stage16(nslots * P / VN, kst, [&](int i) { return K + (uint32_t)(i * VN); });
    stage16(nslots * P / VN, vst, [&](int i) { return V + (uint32_t)(i * VN); });
    const float* ck = a.proj + (crow0 + nrows - m) * ld + h * P;
#pragma unroll
    for (int e = 0; e < FIX; ++e) {
      fk[e] = fv[e] = 0.f;
      if (e * rpp < m) {  // uniform
        const int j = jr + e * rpp;
        if (jr < rpp && j < m) {
          fk[e] = ck[(uint32_t)(sh.off_k + j * ldi + pc)];
          fv[e] = ck[(uint32_t)(sh.off_v + j * ldi + pc)];
        }
      }
    }
  }
  const int64_t count = blk ? 0 : *count_ptr(a.state_pool, sh, slot);
  vm_wait<0>();
  __syncthreads();

  float* op = a.att_part + ((((int64_t)r * nh + h) * a.n_split + sp) * RB) * P;
  float* ml = a.att_ml + ((((int64_t)r * nh + h) * a.n_split + sp) * RB) * 2;
  if (blk) {
    attn_split(sh, RB, ks, true, qs, reinterpret_cast<const float*>(kst), reinterpret_cast<const float*>(vst), pl,
               red, op, ml);
    return;
  }
  const int64_t tot = count + nrows;
  const int valid = (int)(tot < W ? tot : W);
  int nk = valid - k0;
  nk = nk < 0 ? 0 : (nk > ks ? ks : nk);
  if (nk == 0) {
    for (int idx = t; idx < RB * P; idx += RT) st_dev(op + idx, 0.f);
    if (t < RB) {
      st_dev(ml + 2 * t, -INFINITY);
      st_dev(ml + 2 * t + 1, 0.f);
    }
    return;
  }
  if (m > 0) {
    // the slots this round's append overwrites take its rows, rounded as the ring stores them:
    // slot (count + nrows - m + j) mod W holds committed row nrows - m + j
    int lead = mod_w(count, W) + nrows - m;
    while (lead >= W) lead -= W;  // uniform, at most RB / W + 1 steps
#pragma unroll
    for (int e = 0; e < FIX; ++e) {
      const int j = jr + e * rpp;
      if (e * rpp < m && jr < rpp && j < m) {
        int key = lead + j;
        if (key >= W) key -= W;
        key -= k0;
        if (key >= 0 && key < nk) {
          kst[key * P + pc] = from_f32<T>(fk[e]);
          vst[key * P + pc] = from_f32<T>(fv[e]);
        }
      }
    }
    __syncthreads();
  }
  if constexpr (sizeof(T) == 2)
    attn_split_mfma(sh, nk, ks, qs, kst, vst, red, op, ml);
  else
    attn_split(sh, nk, ks, false, qs, kst, vst, pl, red, op, ml);
}

// Merge of one (request, head).  The (max, sum) pairs and the readout are staged in LDS, and each
// thread loads its own 4 consecutive outputs' partials of up to MSPL splits straight into registers,
// all in one memory round trip (device-coherent loads: the partials were written by other
// workgroups, possibly on other XCDs); per (split, row) factors exp(max_s - max) are formed once,
// in parallel, then every output sums its splits.
// Merge LDS (bytes): (max, sum) [ns][RB][2] | factors [ns][RB] | row maxima and sums [2 RB] |
// readout [RB][P].
constexpr int MSPL = 9;                         // splits whose partials one register pass holds
constexpr int MQ = (RB * 256 / 4 + RT - 1) / RT;  // 4-output groups per thread (P <= 256)
template <typename T>
__device__ __forceinline__ void round_merge(const Shape& sh, const RoundArgs& a, int r, int h, char* smem) {
  const int nh = sh.nh, P = sh.P, t = threadIdx.x;
  const int ns = a.n_split;
  const int P4 = P / 4;
  const float* ml = a.att_ml + (((int64_t)r * nh + h) * ns) * RB * 2;
  const float* op = a.att_part + (((int64_t)r * nh + h) * ns) * RB * P;
  float* sml = reinterpret_cast<float*>(smem);
  float* fac = reinterpret_cast<float*>(smem + up1k(ns * RB * 2 * 4));
  float* rowm = reinterpret_cast<float*>(reinterpret_cast<char*>(fac) + up1k(ns * RB * 4));
  float* memv = rowm + 256;
  // the partials of this (request, head): ns * RB * P floats from op, device-coherent buffer loads
  const __amdgpu_buffer_rsrc_t rop = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(op), 0,
                                                                       ns * RB * P * 4, 0x00020000);
  stage16_dev(ns * RB * 2 / 4, sml, [&](int i) { return ml + 4 * i; });
  const Div& dP4 = a.d_p4;
  const float* mrow = a.mem + ((int64_t)r * RB * nh + h) * P;  // row j of the readout: j nh P floats further
  stage16_dev(RB * P4, memv, [&](int i) { const int q = dP4.q(i); return mrow + (uint32_t)(q * nh * P + 4 * (i - q * P4)); });
  T* out = static_cast<T*>(a.o_in);
  bool first = true;  // uniform: the factors are formed after the first round trip
  for (int e = 0; e < MQ; ++e) {
    if (e * RT >= RB * P4) break;  // uniform
    const int q = t + e * RT;      // this thread's group of 4 outputs: row q / P4, columns 4 (q % P4) ..
    const bool mine = q < RB * P4;
    const int j = mine ? dP4.q(q) : 0;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ns; s0 += MSPL) {
      const int nc = ns - s0 < MSPL ? ns - s0 : MSPL;
      f32x4 pv[MSPL];
#pragma unroll
      for (int s = 0; s < MSPL; ++s)
        if (mine && s < nc)
          pv[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rop, 16 * q, ((s0 + s) * RB * P) * 4,
                                                                                   AUX_DEV));
      vm_wait<0>();
      __syncthreads();
      if (first) {
        if (t < RB) {
          float m = -INFINITY;
          for (int s = 0; s < ns; ++s) m = fmaxf(m, sml[(s * RB + t) * 2]);
          rowm[t] = m;
        }
        __syncthreads();
        for (int i = t; i < ns * RB; i += RT) {
          const float ms = sml[2 * i];
          fac[i] = ms == -INFINITY ? 0.f : expf(ms - rowm[i % RB]);
        }
        __syncthreads();
        if (t < RB) {
          float l = 0.f;
          for (int s = 0; s < ns; ++s) l += fac[s * RB + t] * sml[(s * RB + t) * 2 + 1];
          rowm[RB + t] = l;
        }
        __syncthreads();
        first = false;
      }
      if (mine) {
#pragma unroll
        for (int s = 0; s < MSPL; ++s)
          if (s < nc) acc += fac[(s0 + s) * RB + j] * pv[s];
      }
    }
    if (mine) {
      const int pp = 4 * (q - j * P4);
      const float inv = 1.f / rowm[RB + j];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        out[((int64_t)r * RB + j) * sh.dq + h * P + pp + c] = from_f32<T>(acc[c] * inv + memv[j * P + pp + c]);
    }
  }
}

template <typename T, int TMAXG>
__device__ __forceinline__ void round_body(const Shape& sh, const RoundArgs& a, const ReqTable& rt) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  __shared__ int s_last;
  const int nh = sh.nh;
  const int per = a.n_tiles + a.n_split;
  // Block b runs on XCD b % 8: each XCD takes a contiguous range of (request, head, role) items, so
  // the workgroups of one (request, head) share its L2 (the block rows' q and C, read by every
  // split and tile); 64 Qwen3-4B-shaped requests 248 -> 236 us.  Only speed depends on this
  // placement: the hand-over to the merge is device-coherent wherever the workgroups run.  The
  // grid is padded to a multiple of 8.
  const int per_xcd = (int)(gridDim.x / 8);
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (item >= rt.n_req * nh * per) return;
  const int rh = a.d_per.q(item), role = item - rh * per;
  const int r = a.d_nh.q(rh), h = rh - r * nh;
  if (role < a.n_tiles)
    round_tile<T, TMAXG>(sh, a, rt, r, h, role, dsm);
  else
    round_attn<T>(sh, a, rt, r, h, role - a.n_tiles, dsm);

  // count this workgroup in once its stores are complete; the last one of (r, h) merges
  vm_wait<0>();
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(a.counters + rh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == per - 1;
  __syncthreads();
  if (!s_last) return;
  if (a.do_draft) round_merge<T>(sh, a, r, h, dsm);
  if (!a.do_commit) return;
  // the last (r, h) of the request to finish advances its committed count: every workgroup of the
  // request has read the count by then
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(a.counters + rt.n_req * nh + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nh - 1)
    *count_ptr(a.state_pool, sh, rt.slot[r]) += commit_rows(a, rt, r);
}

// ---------------------------------------------------------------------------------------------
// One round with one workgroup per (request, head) (bf16, draft rounds over many pairs): the
// commit / readout of the whole head (round_tile over all P rows, ring append included), then the
// attention of the 8 block rows over the ring window streamed through LDS in chunks of PK = 64
// slots (the next chunk's direct loads in flight while the current one is multiplied), with a
// running softmax per wave on bf16 matrix cores, then the block keys, and the output written
// directly: no partial results, no merge.
//   scores:  wave w takes slots 16 w .. 16 w + 15 of every chunk: S^T = K Q^T (A = 16 slots x 16
//            dims of K, B = 16 dims x 16 queries as (hi, lo) bf16 pairs; rows 8..15 repeat 0..7);
//            lane l holds slots 16 w + 4 (l / 16) + r (r = 0..3) of query l % 16.
//   values:  O^T += V^T P^T (A = 16 dims x 16 slots of V, four 2-byte LDS reads per lane; B = those
//            probabilities as (hi, lo) pairs), so lane l's accumulators are dimensions
//            16 c + 4 (l / 16) + r of query l % 16, and the running maximum rescales them in place.
//   The ring rows this round's append overwrites are read from the projection instead (rounded
//   as the ring stores them), so a chunk's contents do not depend on whether the append's stores
//   have landed.  Rows past the window's valid slots are masked: their scores replaced by -inf,
//   their value rows zeroed.
constexpr int PK = 64;  // ring slots per chunk: 16 per wave
template <typename T>
struct PairLds {  // byte offsets: [tile buffers 0, 1 | buffer 2 or the commit region] then q, fk, fv, bk, bv, memv, scratch
  int commit, q, fk, fv, bk, bv, memv, red, total;
  __host__ __device__ PairLds(const Shape& sh, int commit_bytes, bool m2) {
    // the Mamba-2 kernel keeps its ring tiles in registers; the other streams them through LDS
    const int slot = 4 * 2 * 16 * sh.P * (int)sizeof(T);  // one tile of K and V for each of the four waves
    commit = m2 ? 0 : 2 * slot;  // LDS buffers 0 and 1 fill while the commit runs
    const int a = m2 ? commit_bytes : commit + (commit_bytes > slot ? commit_bytes : slot);
    int o = up1k(a);
    const int rows = up1k(RB * sh.P * 4);
    q = o; o += rows;
    fk = o; o += rows;
    fv = o; o += rows;
    bk = o; o += rows;
    bv = o; o += rows;
    memv = o; o += m2 ? rows : 0;
    red = o; o += 4 * 256;
    total = o;
  }
};
// Commit region of the Mamba-2 pair kernel: B of the committed rows [RB][N] | C of the block rows
// [RB][N] | the waves' readout partials [4][P][RB], all fp32.
__host__ __device__ constexpr int m2_commit_bytes(int P, int N) { return 2 * up1k(RB * N * 4) + up1k(4 * P * RB * 4); }

// NPC: dimension tiles of a head (P = 16 NPC) fixed at compile time, or 0 (P from the shape).
// M2: the Mamba-2 commit and readout on fp32 matrix cores (NBW column blocks of H per wave) instead
// of round_tile (which also serves the gated delta rule and the last-W memory).
template <typename T, int NPC, bool M2, int NBW>
__device__ __forceinline__ void pair_body(const Shape& sh, const RoundArgs& a, const ReqTable& rt, int r, int h,
                                          char* smem, int commit_bytes) {
  const int nh = sh.nh, P = NPC ? 16 * NPC : sh.P, W = sh.W, N = sh.N, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int P4 = P / 4, npc = NPC ? NPC : P / 16;
  const PairLds<T> L(sh, commit_bytes, M2);
  float* qs = reinterpret_cast<float*>(smem + L.q);
  float* fk = reinterpret_cast<float*>(smem + L.fk);
  float* fv = reinterpret_cast<float*>(smem + L.fv);
  float* bk = reinterpret_cast<float*>(smem + L.bk);
  float* bv = reinterpret_cast<float*>(smem + L.bv);
  float* red = reinterpret_cast<float*>(smem + L.red);  // [4][16] maxima | [4][16] sums | [8][8] block scores | factors
  const int slot = rt.slot[r];
  const int nrows = a.do_commit ? commit_rows(a, rt, r) : 0;
  const int m = nrows < W ? nrows : W;  // committed rows that land in the ring
  const int64_t crow0 = a.dev_rows ? (int64_t)RB * r : rt.row0[r];
  const int64_t brow0 = a.blk_row0 + (int64_t)r * RB;
  const int ldi = (int)a.ld;
  const Div& dP4 = a.d_p4;
  // the attention's inputs go out with the commit tile's loads (its wait covers them)
  const float* bq = a.proj + brow0 * a.ld + h * P;
  const float* cq = a.proj + (crow0 + nrows - m) * a.ld + h * P;
  stage16(RB * P4, qs, [&](int i) { const int q = dP4.q(i); return bq + (uint32_t)(sh.off_q + q * ldi + 4 * (i - q * P4)); });
  stage16(RB * P4, bk, [&](int i) { const int q = dP4.q(i); return bq + (uint32_t)(sh.off_k + q * ldi + 4 * (i - q * P4)); });
  stage16(RB * P4, bv, [&](int i) { const int q = dP4.q(i); return bq + (uint32_t)(sh.off_v + q * ldi + 4 * (i - q * P4)); });
  stage16(m * P4, fk, [&](int i) { const int q = dP4.q(i); return cq + (uint32_t)(sh.off_k + q * ldi + 4 * (i - q * P4)); });
  stage16(m * P4, fv, [&](int i) { const int q = dP4.q(i); return cq + (uint32_t)(sh.off_v + q * ldi + 4 * (i - q * P4)); });
  const int64_t count = *count_ptr(a.state_pool, sh, slot);
  float* memv = reinterpret_cast<float*>(smem + L.memv);  // [RB][P] readout (M2)
  // the first two ring tiles of every wave go out with these loads (see the attention below)
  const T* Kr = ring_ptr<T>(a.state_pool, sh, slot, sh.st_k, h);
  const T* Vr = ring_ptr<T>(a.state_pool, sh, slot, sh.st_v, h);
  const int tb = 16 * P * (int)sizeof(T);  // bytes of one 16-slot tile of K or V
  const int NI = (P + 31) / 32;            // 1 KiB loads per tile (2 P 16-byte pieces)
  auto tbuf = [&](int c) { return smem + ((c % 3) * 4 + wave) * 2 * tb; };
  auto issue = [&](int c) {
    // rows of this wave's tile that lie inside the ring (at least one: a tile past the ring
    // re-reads the ring's last row); the slots' validity is decided later, from the count
    const int row0 = PK * c + 16 * wave < W ? PK * c + 16 * wave : W - 1;
    const int avail = W - row0 < 16 ? W - row0 : 16;
    const int lim = avail * P * (int)sizeof(T) - 16;  // last whole 16-byte piece of those rows
    const char* ks = reinterpret_cast<const char*>(Kr + (int64_t)row0 * P);
    const char* vs = reinterpret_cast<const char*>(Vr + (int64_t)row0 * P);
    char* dk = tbuf(c);
#pragma unroll 1
    for (int n = 0; n < NI; ++n) {
      // lanes past the tile's 2 P pieces stay idle (the last load keeps at least 32 lanes)
      const int b = 1024 * n + 16 * lane;
      if (b < tb) {
        lds_dma16(ks + (uint32_t)(b < lim ? b : lim), dk + 1024 * n);
        lds_dma16(vs + (uint32_t)(b < lim ? b : lim), dk + tb + 1024 * n);
      }
    }
  };
  if constexpr (!M2) {
    issue(0);
    issue(1);
  }
  char* creg = smem + L.commit;
  if constexpr (!M2) {
    round_tile<T, WIDE_PASSES>(sh, a, rt, r, h, 0, creg);  // its readout goes to a.mem (device scope)
  } else {
    // ---- Mamba-2 commit and readout on fp32 matrix cores (16x16x4: exact products, fp32 sums).
    // H^T is held in 16 x 16 blocks (state columns n x rows p of H) in the accumulator layout:
    // lane (li, g) holds H[16 pb + li][16 nb + 4 g + r], r = 0..3, one 16-byte piece of a row of H,
    // so a block loads and stores with one access per lane.  Wave w owns column blocks w, w + 4,
    // ... of every row block.
    //   commit:  H^T <- dec H^T + B^T (w x)  (A: lane holds B_t[16 nb + li] for row t = 4 s + g;
    //            B: w_t x_t[16 pb + li]; two steps of four committed rows).
    //   readout: Y^T[p][j] = sum_n H[p][n] C_j[n], four steps per block with A = the lane's
    //            register r (row li, column 16 nb + 4 g + r) and B = C_li[16 nb + 4 g + r]; the waves'
    //            partial sums over their columns meet in LDS.
    const int NB = N / 16;
    constexpr int PB = NPC;
    float* Bl = reinterpret_cast<float*>(creg);
    float* Cl = reinterpret_cast<float*>(creg + up1k(RB * N * 4));
    float* part = reinterpret_cast<float*>(creg + 2 * up1k(RB * N * 4));  // [4][P][RB]
    float* wl = red;  // weights of the committed rows, the old state's decay at RMAXC
    const int grp = h / (nh / sh.G);
    float* Hh = h_ptr(a.state_pool, sh, slot, h);
    f32x4 hreg[PB][NBW];
#pragma unroll
    for (int pb = 0; pb < PB; ++pb)
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        const int nb = wave + 4 * b;
        hreg[pb][b] = nb < NB ? *reinterpret_cast<const f32x4*>(Hh + (16 * pb + li) * N + 16 * nb + 4 * g)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    const int N4 = N / 4;
    const float* cb = a.proj + crow0 * a.ld + sh.off_b + grp * N;
    const float* bc = a.proj + brow0 * a.ld + sh.off_c + grp * N;
    stage16(nrows * N4, Bl, [&](int i) { const int q = a.d_tpr.q(i); return cb + (uint32_t)(q * ldi + 4 * (i - q * N4)); });
    stage16(RB * N4, Cl, [&](int i) { const int q = a.d_tpr.q(i); return bc + (uint32_t)(q * ldi + 4 * (i - q * N4)); });
    const float raw = t < nrows ? a.proj[(crow0 + t) * a.ld + sh.off_dt + h] : 0.f;
    vm_wait<0>();
    __syncthreads();
    if (t < 64) {
      // w_t = dt_t exp(sum_{tau > t} dt_tau A) and the decay exp(sum_t dt_t A); lane t holds row t
      const float A = -expf(a.a_log[h]);
      const float dt = t < nrows ? softplus_f(raw + a.dt_bias[h]) : 0.f;
      const float ell = dt * A;
      float inc = ell;
#pragma unroll
      for (int o = 1; o < RMAXC; o <<= 1) {
        const float v = __shfl_down(inc, o, 64);
        if (t + o < RMAXC) inc += v;
      }
      if (t < nrows) wl[t] = dt * expf(inc - ell);
      if (t == 0) wl[RMAXC] = expf(inc);
    }
    __syncthreads();
    if (nrows > 0) {
      const float dec = wl[RMAXC];
      float bw[2][PB];  // w_t x_t[16 pb + li] for t = 4 s + g
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int tt = 4 * s2 + g;
#pragma unroll
        for (int pb = 0; pb < PB; ++pb) bw[s2][pb] = tt < nrows ? wl[tt] * fv[tt * P + 16 * pb + li] : 0.f;
      }
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        const int nb = wave + 4 * b;
        if (nb < NB) {  // uniform
          float ba[2];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int tt = 4 * s2 + g;
            ba[s2] = tt < nrows ? Bl[tt * N + 16 * nb + li] : 0.f;
          }
#pragma unroll
          for (int pb = 0; pb < PB; ++pb) {
            f32x4 acc = hreg[pb][b] * dec;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ba[0], bw[0][pb], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ba[1], bw[1][pb], acc, 0, 0, 0);
            hreg[pb][b] = acc;
            *reinterpret_cast<f32x4*>(Hh + (16 * pb + li) * N + 16 * nb + 4 * g) = acc;
          }
        }
      }
    }
    // readout partials of this wave's columns
#pragma unroll
    for (int pb = 0; pb < PB; ++pb) {
      f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        const int nb = wave + 4 * b;
        if (nb < NB) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(hreg[pb][b][rr], Cl[(li & 7) * N + 16 * nb + 4 * g + rr], y, 0, 0, 0);
        }
      }
      // lane (li, g) holds Y^T[16 pb + 4 g + rr][li]; queries li < RB are the block rows
      if (li < RB)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) part[(wave * P + 16 * pb + 4 * g + rr) * RB + li] = y[rr];
    }
    __syncthreads();
    const float D = a.d_skip[h];
    for (int i = t; i < RB * P; i += RT) {
      const int j = i / P, p = i - j * P;  // P is a compile-time constant here
      memv[i] = part[(0 * P + p) * RB + j] + part[(1 * P + p) * RB + j] + part[(2 * P + p) * RB + j] +
                part[(3 * P + p) * RB + j] + D * bv[j * P + p];
    }
    // ring append of this round's rows (the last m), from the staged projection rows
    if (nrows > 0) {
      T* Kw = ring_ptr<T>(a.state_pool, sh, slot, sh.st_k, h);
      T* Vw = ring_ptr<T>(a.state_pool, sh, slot, sh.st_v, h);
      int s0 = mod_w(count, W) + nrows - m;
      while (s0 >= W) s0 -= W;
      for (int j = 0; j < m; ++j) {  // uniform
        const int sl = s0 + j >= W ? s0 + j - W : s0 + j;
        for (int p = t; p < P; p += RT) {
          Kw[sl * P + p] = from_f32<T>(fk[j * P + p]);
          Vw[sl * P + p] = from_f32<T>(fv[j * P + p]);
        }
      }
    }
  }
  __syncthreads();  // the commit region is free

  // ---- block keys: wave 0, lane = 8 q + key, exact fp32 scores (before q turns into bf16 pairs)
  const float scale = rsqrtf((float)P);
  float* sb = red + 128;
  if (wave == 0) {
    const int q = lane >> 3, key = lane & 7;
    float acc = 0.f;
    for (int p = 0; p < P; p += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(qs + q * P + p);
      const f32x4 y = *reinterpret_cast<const f32x4*>(bk + key * P + p);
      acc = fmaf(x[0], y[0], acc);
      acc = fmaf(x[1], y[1], acc);
      acc = fmaf(x[2], y[2], acc);
      acc = fmaf(x[3], y[3], acc);
    }
    sb[lane] = (!sh.cross && key != q) ? -INFINITY : acc * scale;
  }
  // ---- queries -> (hi, lo) bf16 pairs in place
  constexpr int QE = RB * 256 / RT;
  float qv[QE];
#pragma unroll
  for (int e = 0; e < QE; ++e) qv[e] = t + e * RT < RB * P ? qs[t + e * RT] : 0.f;
  __syncthreads();
  short* qh = reinterpret_cast<short*>(qs);
  short* ql = qh + RB * P;
#pragma unroll
  for (int e = 0; e < QE; ++e) {
    const int i = t + e * RT;
    if (i < RB * P) {
      const short hb = bf16_bits(qv[e]);
      qh[i] = hb;
      ql[i] = bf16_bits(qv[e] - bf16_val(hb));
    }
  }

  // ---- the ring window after this round's append: wave w streams slots 64 c + 16 w .. + 15 of
  // every chunk c through three LDS buffers of its own (two tiles in flight while one is
  // multiplied; tiles 0 and 1 went out with the commit's loads); a tile is NI = ceil(P / 32) direct
  // loads per operand for every wave and chunk (addresses past the ring clamped to its rows), so
  // the waits are fixed counts and the waves never meet.
  const int64_t tot = count + nrows;
  const int valid = (int)(tot < W ? tot : W);
  const int nch = (valid + PK - 1) / PK;
  int lead = mod_w(count, W) + nrows - m;  // slot of committed row nrows - m
  while (lead >= W) lead -= W;
  const int qrow = (li & 7) * P;
  float mrun = -INFINITY, lrun = 0.f;
  f32x4 o[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (M2) {
    // Ring tiles straight into registers: lane (li, g) of wave w loads slot 64 c + 16 w + li,
    // 16 bytes per 32 dimensions (dimensions 32 cc + 8 g .. + 7, the 16x16x32 operand layout) and
    // 8 bytes for a last run of 16 (dimensions + 4 g .. + 3, 16x16x16).  K is the A operand of the
    // scores as it stands; V goes through one exact product with a 0/1 matrix per 16 dimensions,
    // D = V I, whose accumulator layout (lane: dimension li, slots 4 g .. 4 g + 3) is the A operand
    // of O^T += V^T P^T.  The next tile loads while one is multiplied (two register sets, rotated by
    // unrolling): 118 VGPRs and four workgroups per CU measured faster than two tiles in flight
    // with three per CU (119 against 127 us at 64 Qwen3-4B-shaped requests).
    constexpr int NC = NPC / 2, TAIL = NPC % 2;  // 32-dimension runs, and a last run of 16
    struct Tile {
      bf16x8 k[NC], v[NC];
      s16x4 kt, vt;
    };
    vm_wait<0>();     // the commit's stores are out
    __syncthreads();  // the q pairs are published
    bf16x8 idf[2];
    s16x4 idt;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) idf[hh][e] = static_cast<bf16>(8 * g + e == 16 * hh + li ? 1.f : 0.f);
#pragma unroll
    for (int e = 0; e < 4; ++e) idt[e] = bf16_bits(4 * g + e == li ? 1.f : 0.f);
    const T* Kr2 = ring_ptr<T>(a.state_pool, sh, slot, sh.st_k, h);
    const T* Vr2 = ring_ptr<T>(a.state_pool, sh, slot, sh.st_v, h);
    auto load = [&](int c, Tile& d) __attribute__((always_inline)) {
      int row = PK * c + 16 * wave + li;
      row = row < W ? row : W - 1;  // rows past the ring re-read its last row (masked below)
      const bf16* kp = reinterpret_cast<const bf16*>(Kr2) + row * P;
      const bf16* vp = reinterpret_cast<const bf16*>(Vr2) + row * P;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        d.k[cc] = *reinterpret_cast<const bf16x8*>(kp + 32 * cc + 8 * g);
        d.v[cc] = *reinterpret_cast<const bf16x8*>(vp + 32 * cc + 8 * g);
      }
      if constexpr (TAIL) {
        d.kt = *reinterpret_cast<const s16x4*>(kp + 32 * NC + 4 * g);
        d.vt = *reinterpret_cast<const s16x4*>(vp + 32 * NC + 4 * g);
      }
    };
    auto step = [&](int c, Tile& cur, Tile& nxt) __attribute__((always_inline)) {
      if (c + 1 < nch) load(c + 1, nxt);
      const int nv = valid - PK * c < PK ? valid - PK * c : PK;
      const int nw = nv - 16 * wave < 16 ? nv - 16 * wave : 16;  // valid slots of this wave's tile
      if (nw <= 0) return;                                       // uniform per wave
      // this round's committed rows replace the slots the append overwrites; value rows past the
      // valid ones are zeroed (a zero probability times a NaN would not be zero)
      const int myslot = PK * c + 16 * wave + li;
      for (int j = 0; j < m; ++j) {  // uniform
        int sl = lead + j;
        if (sl >= W) sl -= W;
        if (sl == myslot) {
          const float* fkr = fk + j * P;
          const float* fvr = fv + j * P;
#pragma unroll
          for (int cc = 0; cc < NC; ++cc)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              cur.k[cc][e] = static_cast<bf16>(fkr[32 * cc + 8 * g + e]);
              cur.v[cc][e] = static_cast<bf16>(fvr[32 * cc + 8 * g + e]);
            }
          if constexpr (TAIL)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              cur.kt[e] = bf16_bits(fkr[32 * NC + 4 * g + e]);
              cur.vt[e] = bf16_bits(fvr[32 * NC + 4 * g + e]);
            }
        }
      }
      if (li >= nw) {
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) cur.v[cc] = bf16x8{};
        cur.vt = s16x4{0, 0, 0, 0};
      }
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const bf16x8 qb = *reinterpret_cast<const bf16x8*>(qh + qrow + 32 * cc + 8 * g);
        const bf16x8 qc = *reinterpret_cast<const bf16x8*>(ql + qrow + 32 * cc + 8 * g);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[cc], qb, sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[cc], qc, sacc, 0, 0, 0);
      }
      if constexpr (TAIL) {
        const s16x4 qb = *reinterpret_cast<const s16x4*>(qh + qrow + 32 * NC + 4 * g);
        const s16x4 qc = *reinterpret_cast<const s16x4*>(ql + qrow + 32 * NC + 4 * g);
        sacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cur.kt, qb, sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cur.kt, qc, sacc, 0, 0, 0);
      }
      float sv[4], cm = -INFINITY;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        sv[rr] = 4 * g + rr < nw ? sacc[rr] * scale : -INFINITY;
        cm = fmaxf(cm, sv[rr]);
      }
      cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
      cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
      const float mnew = fmaxf(mrun, cm);  // finite: the tile's first slot is valid
      const float alpha = mrun == -INFINITY ? 0.f : __expf(mrun - mnew);
      mrun = mnew;
      s16x4 ph, pl;
      float ps = 0.f;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float pv = sv[rr] == -INFINITY ? 0.f : __expf(sv[rr] - mnew);
        ps += pv;
        const short hb = bf16_bits(pv);
        ph[rr] = hb;
        pl[rr] = bf16_bits(pv - bf16_val(hb));
      }
      lrun = lrun * alpha + ps;
      auto pv_run = [&](int d, const f32x4& tr) __attribute__((always_inline)) {
        s16x4 va;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) va[rr] = bf16_bits(tr[rr]);  // exact: the values are bf16
        o[d] *= alpha;
        o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph, o[d], 0, 0, 0);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl, o[d], 0, 0, 0);
      };
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          pv_run(2 * cc + hh,
                 __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.v[cc], idf[hh], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0));
      if constexpr (TAIL)
        pv_run(2 * NC, __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cur.vt, idt, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0));
    };
    Tile t0, t1;
    if (nch > 0) load(0, t0);
    for (int c = 0; c < nch; c += 2) {
      step(c, t0, t1);
      if (c + 1 < nch) step(c + 1, t1, t0);
    }
  } else {
  auto wait_tiles = [&](int pending) {  // this wave's loads of `pending` later tiles may stay out
    const int n = pending * 2 * NI;
    if (n >= 16) vm_wait<16>();
    else if (n >= 12) vm_wait<12>();
    else if (n >= 8) vm_wait<8>();
    else if (n >= 6) vm_wait<6>();
    else if (n >= 4) vm_wait<4>();
    else if (n >= 2) vm_wait<2>();
    else vm_wait<0>();
  };
  vm_wait<0>();     // the commit's stores are out of the count: only tile loads from here on
  __syncthreads();  // the commit region (buffer 2) is free; the q pairs are published
  for (int c = 0; c < nch; ++c) {
    if (c + 2 < nch) issue(c + 2);  // buffer (c + 2) % 3 held tile c - 1, done above
    wait_tiles(nch - 1 - c < 2 ? nch - 1 - c : 2);
    const int nv = valid - PK * c < PK ? valid - PK * c : PK;
    const int nw = nv - 16 * wave < 16 ? nv - 16 * wave : 16;  // valid slots of this wave's tile
    if (nw <= 0) continue;          // uniform per wave
    T* kc = reinterpret_cast<T*>(tbuf(c));
    T* vc = reinterpret_cast<T*>(tbuf(c) + tb);
    // this round's committed rows replace the slots the append overwrites; value rows past the
    // valid ones are zeroed (a zero probability times a NaN would not be zero)
    for (int j = 0; j < m; ++j) {  // uniform
      int sl = lead + j;
      if (sl >= W) sl -= W;
      sl -= PK * c + 16 * wave;
      if (sl >= 0 && sl < nw)
        for (int p = lane; p < P; p += 64) {
          kc[sl * P + p] = from_f32<T>(fk[j * P + p]);
          vc[sl * P + p] = from_f32<T>(fv[j * P + p]);
        }
    }
    if (nw < 16)
      for (int i2 = lane; i2 < (16 - nw) * P; i2 += 64) vc[nw * P + i2] = from_f32<T>(0.f);
    // scores of slots PK c + 16 wave + 4 g + r for query li (the wave's own LDS writes are ordered
    // before its reads)
    const short* kr = reinterpret_cast<const short*>(kc) + li * P + 4 * g;
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int cc = 0; cc < npc; ++cc) {
      const s16x4 ka = *reinterpret_cast<const s16x4*>(kr + 16 * cc);
      const s16x4 qb = *reinterpret_cast<const s16x4*>(qh + qrow + 16 * cc + 4 * g);
      const s16x4 qc = *reinterpret_cast<const s16x4*>(ql + qrow + 16 * cc + 4 * g);
      sacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, qb, sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, qc, sacc, 0, 0, 0);
    }
    float sv[4], cm = -INFINITY;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      sv[rr] = 4 * g + rr < nw ? sacc[rr] * scale : -INFINITY;
      cm = fmaxf(cm, sv[rr]);
    }
    cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
    cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
    const float mnew = fmaxf(mrun, cm);  // finite: the tile's first slot is valid
    const float alpha = mrun == -INFINITY ? 0.f : __expf(mrun - mnew);
    mrun = mnew;
    s16x4 ph, pl;
    float ps = 0.f;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float pv = sv[rr] == -INFINITY ? 0.f : __expf(sv[rr] - mnew);
      ps += pv;
      const short hb = bf16_bits(pv);
      ph[rr] = hb;
      pl[rr] = bf16_bits(pv - bf16_val(hb));
    }
    lrun = lrun * alpha + ps;
    const short* vr = reinterpret_cast<const short*>(vc) + 4 * g * P + li;
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) {
      if (cc < npc) {
        s16x4 va;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) va[rr] = vr[rr * P + 16 * cc];
        o[cc] *= alpha;
        o[cc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph, o[cc], 0, 0, 0);
        o[cc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl, o[cc], 0, 0, 0);
      }
    }
  }
  }
  // ---- the waves' (max, sum, O) and the block keys
  lrun += __shfl_xor(lrun, 16, 64);
  lrun += __shfl_xor(lrun, 32, 64);
  if (g == 0) {
    red[wave * 16 + li] = mrun;
    red[64 + wave * 16 + li] = lrun;
  }
  vm_wait<0>();     // this thread's readout stores (round_tile) are complete before the reads below
  __syncthreads();  // every chunk read is done: the chunk region takes the waves' O
  float* ob = reinterpret_cast<float*>(smem);  // [4][RB][P]
  if (li < RB) {
#pragma unroll
    for (int cc = 0; cc < 16; ++cc)
      if (cc < npc)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) ob[(wave * RB + li) * P + 16 * cc + 4 * g + rr] = o[cc][rr];
  }
  float* fac = red + 192;  // [RB][8]: wave factors 0..3, 1 / sum at 4
  float* fbk = red + 128;  // block scores -> block factors in place
  if (t < RB) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red[w * 16 + t]);
#pragma unroll
    for (int k = 0; k < RB; ++k) M = fmaxf(M, sb[t * RB + k]);
    float Ls = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = red[w * 16 + t];
      const float f = mw == -INFINITY ? 0.f : __expf(mw - M);
      fac[t * 8 + w] = f;
      Ls += f * red[64 + w * 16 + t];
    }
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const float sk = sb[t * RB + k];
      const float f = sk == -INFINITY ? 0.f : __expf(sk - M);
      fbk[t * RB + k] = f;
      Ls += f;
    }
    fac[t * 8 + 4] = 1.f / Ls;
  }
  __syncthreads();
  T* out = static_cast<T*>(a.o_in);
  for (int i = t; i < RB * P; i += RT) {
    const int q = NPC ? i / P : a.d_p.q(i), p = i - q * P;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) v += fac[q * 8 + w] * ob[(w * RB + q) * P + p];
#pragma unroll
    for (int k = 0; k < RB; ++k) v += fbk[q * RB + k] * bv[k * P + p];
    float mem;
    if constexpr (M2)
      mem = memv[i];
    else
      mem = __hip_atomic_load(a.mem + (((int64_t)r * RB + q) * nh + h) * P + p, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    out[((int64_t)r * RB + q) * sh.dq + h * P + p] = from_f32<T>(v * fac[q * 8 + 4] + mem);
  }
}

// One (request, head) per workgroup; the last head of a request to finish advances its count.
template <typename T, int NPC, bool M2, int NBW>
__global__ void __launch_bounds__(RT) __attribute__((amdgpu_waves_per_eu(M2 ? 4 : 2))) k_round_pair(Shape sh, RoundArgs a,
                                                                                           ReqTable rt, int commit_bytes) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  const int per_xcd = (int)(gridDim.x / 8);
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (item >= rt.n_req * sh.nh) return;
  const int r = a.d_nh.q(item), h = item - r * sh.nh;
  pair_body<T, NPC, M2, NBW>(sh, a, rt, r, h, dsm, commit_bytes);
  if (!a.do_commit) return;
  vm_wait<0>();
  __syncthreads();
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(a.counters + rt.n_req * sh.nh + r, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
          sh.nh - 1)
    *count_ptr(a.state_pool, sh, rt.slot[r]) += commit_rows(a, rt, r);
}

// Tiles of up to MID_PASSES row passes (the narrow layout): the register budget (80 VGPRs) and
// the LDS of the attention splits keep six workgroups on a CU (64 Qwen3-4B-shaped requests: 221
// against 233 us with five workgroups and three-pass tiles).
template <typename T, int TMAXG>
__global__ void __launch_bounds__(RT) __attribute__((amdgpu_waves_per_eu(6))) k_round(Shape sh, RoundArgs a,
                                                                                     ReqTable rt) {
  round_body<T, TMAXG>(sh, a, rt);
}
// Tiles of up to WIDE_PASSES row passes (the wide layout).
template <typename T, int TMAXG>
__global__ void __launch_bounds__(RT) k_round_wide(Shape sh, RoundArgs a, ReqTable rt) {
  round_body<T, TMAXG>(sh, a, rt);
}

template <typename T>
__global__ void __launch_bounds__(256) k_ring_append(Shape sh, char* pool, ReqTable rt, const T* __restrict__ k,
                                                     int64_t ld_k, const T* __restrict__ vT, int64_t ld_v,
                                                     const float* __restrict__ dtT, int64_t ld_dt) {
  const int nh = sh.nh, P = sh.P, W = sh.W;
  const int r = blockIdx.x / nh, h = blockIdx.x % nh;
  const int64_t n = rt.row0[r + 1] - rt.row0[r];
  if (n <= 0) return;
  const int64_t m = n < W ? n : W;
  // k rows of this request sit after those of the earlier requests (the last min(n, W) each)
  int64_t krow = 0;
  for (int q = 0; q < r; ++q) {
    const int64_t nq = rt.row0[q + 1] - rt.row0[q];
    krow += nq < W ? nq : W;
  }
  const int slot = rt.slot[r];
  const int64_t count = *count_ptr(pool, sh, slot);
  T* K = ring_ptr<T>(pool, sh, slot, sh.st_k, h);
  T* V = ring_ptr<T>(pool, sh, slot, sh.st_v, h);
  for (int64_t idx = (int64_t)blockIdx.y * 256 + threadIdx.x; idx < m * P; idx += (int64_t)gridDim.y * 256) {
    const int64_t j = idx / P;
    const int pp = (int)(idx % P);
    const int64_t s = (count + n - m + j) % W;
    const int64_t tok = n - m + j;  // token of the request in the time-blocked v
    K[s * P + pp] = k[(krow + j) * ld_k + h * P + pp];
    V[s * P + pp] = vT[(rt.blk0[r] + tok / HYF_TBLK) * ld_v + tile_off<T>(h * P + pp, (int)(tok % HYF_TBLK))];
  }
  if (!sh.lastw) return;
  // the last-W memory's rings: the raw step of head h, and (one head per group) the group's B row
  char* blob = pool + (int64_t)slot * sh.st_bytes;
  float* DTr = reinterpret_cast<float*>(blob + sh.st_dt) + (int64_t)h * W;
  T* Br = reinterpret_cast<T*>(blob + sh.st_b);
  const int N = sh.N, grp = h / (sh.nh / sh.G);
  for (int64_t j = (int64_t)blockIdx.y * 256 + threadIdx.x; j < m; j += (int64_t)gridDim.y * 256) {
    const int64_t s = (count + n - m + j) % W, tok = n - m + j;
    DTr[s] = dtT[(rt.blk0[r] + tok / HYF_TBLK) * ld_dt + (int64_t)h * HYF_TBLK + tok % HYF_TBLK];
  }
  if (h % (sh.nh / sh.G) != 0) return;
  for (int64_t idx = (int64_t)blockIdx.y * 256 + threadIdx.x; idx < m * N; idx += (int64_t)gridDim.y * 256) {
    const int64_t j = idx / N;
    const int nn = (int)(idx % N);
    const int64_t s = (count + n - m + j) % W, tok = n - m + j;
    Br[s * sh.gn + grp * N + nn] =
        vT[(rt.blk0[r] + tok / HYF_TBLK) * ld_v + tile_off<T>(sh.dq + grp * N + nn, (int)(tok % HYF_TBLK))];
  }
}

// The last-W memory's rescan input.  Window position j (0 .. W - 1) holds the committed row in ring
// slot (count - W + j) mod W when j >= W - min(count, W), else padding (zeros).  One workgroup per
// (request, time block of the window, e) where e < nh is head e (its x rows, its raw steps, and a
// share of its H, zeroed) and e = nh + g is group g's B rows.  Each thread writes whole 16-byte
// chunks of the tiled layout (VN tokens of one feature, consecutive threads on consecutive
// features, so the ring reads of a wave are contiguous rows and the writes fill 1 KiB tiles in
// lane order); slot arithmetic stays 32-bit (count mod W taken once).
template <typename T>
__global__ void __launch_bounds__(256) k_lastw_gather(Shape sh, char* pool, ReqTable rt, T* __restrict__ vb,
                                                      int64_t ld_vb, float* __restrict__ dtT, int64_t ld_dt,
                                                      int nblk) {
  typedef typename Vec16<T>::type V;
  constexpr int VN = Vec16<T>::n;
  const int nh = sh.nh, P = sh.P, N = sh.N, W = sh.W;
  const int ne = nh + sh.G;
  const int blk = (int)(blockIdx.x % nblk);
  const int e = (int)((blockIdx.x / nblk) % ne);
  const int r = (int)(blockIdx.x / (nblk * ne));
  char* blob = pool + (int64_t)rt.slot[r] * sh.st_bytes;
  const int64_t count = *reinterpret_cast<const int64_t*>(blob);
  const int pad = count < W ? W - (int)count : 0;
  const int c = (int)(count % W);
  const int j0 = blk * HYF_TBLK;
  const int jn = min(W - j0, HYF_TBLK);  // window positions in this block
  T* dst = vb + (int64_t)(rt.blk0[r] + blk) * ld_vb;
  auto ring_slot = [&](int j) {
    const int q = c + j;
    return q >= W ? q - W : q;
  };
  // rows: the ring of this head's x (pitch P) or of the group's B (pitch gn, offset g N)
  const bool is_b = e >= nh;
  const int nf = is_b ? N : P;
  const int64_t f0 = is_b ? (int64_t)sh.dq + (int64_t)(e - nh) * N : (int64_t)e * P;
  const T* src = is_b ? reinterpret_cast<const T*>(blob + sh.st_b) + (int64_t)(e - nh) * N
                      : reinterpret_cast<const T*>(blob + sh.st_v) + (int64_t)e * W * P;
  const int pitch = is_b ? sh.gn : P;
  const int nch = nf * (HYF_TBLK / VN);
  for (int i = threadIdx.x; i < nch; i += 256) {
    const int f = i % nf, tc = i / nf;
    V v;
#pragma unroll
    for (int u = 0; u < VN; ++u) {
      const int jj = tc * VN + u, j = j0 + jj;
      v[u] = jj < jn && j >= pad ? src[(int64_t)ring_slot(j) * pitch + f] : from_f32<T>(0.f);
    }
    *reinterpret_cast<V*>(dst + tile_off<T>(f0 + f, tc * VN)) = v;
  }
  if (is_b) return;
  const int h = e;
  const float* DTr = reinterpret_cast<const float*>(blob + sh.st_dt) + (int64_t)h * W;
  for (int jj = threadIdx.x; jj < HYF_TBLK; jj += 256) {
    const int j = j0 + jj;
    dtT[(int64_t)(rt.blk0[r] + blk) * ld_dt + (int64_t)h * HYF_TBLK + jj] = jj < jn && j >= pad ? DTr[ring_slot(j)] : 0.f;
  }
  // this block's share of H (P N / 4 16-byte words over the nblk blocks of the head)
  f32x4* H = reinterpret_cast<f32x4*>(blob + sh.st_h) + (int64_t)h * P * N / 4;
  const int words = P * N / 4, share = (words + nblk - 1) / nblk;
  const int w1 = min(words, (blk + 1) * share);
  for (int i = blk * share + threadIdx.x; i < w1; i += 256) H[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

__global__ void k_bump_counts(char* pool, Shape sh, ReqTable rt) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < rt.n_req) *count_ptr(pool, sh, rt.slot[r]) += rt.row0[r + 1] - rt.row0[r];
}

__global__ void k_zero(uint32_t* p, uint64_t words) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ void k_reset_states(char* pool, Shape sh, ReqTable rt) {
  const int r = blockIdx.y;
  uint32_t* p = reinterpret_cast<uint32_t*>(pool + (int64_t)rt.slot[r] * sh.st_bytes);
  const uint64_t words = sh.st_bytes / 4;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Layout of a round launch: rows of H per commit tile and keys per attention split.  The narrow
// layout (tiles of one row pass, 64-key splits) spreads one head over ~20 small workgroups; it is
// the faster one at every Qwen3-4B-shaped batch measured (64 requests: 300 us against 358 us for
// the wide one).  The wide layout (tiles of up to WIDE_PASSES row passes, splits of up to 128 keys)
// moves more bytes per workgroup and is taken for heads of 128 or more dimensions over many
// (request, head) pairs, where it measured faster (16 Phi-4-shaped requests: 178 us against 193 us).
constexpr int WIDE_MIN_PAIRS = 256;
constexpr int WIDE_MIN_P = 128;
constexpr int WIDE_KS = 128;
static int attn_lds(const Shape& sh, int esz, int ks) {
  // the block split keeps fp32 k, v rows where the ring splits keep ks ring slots
  const int kv = up1k(ks * sh.P * esz) > up1k(RB * sh.P * 4) ? up1k(ks * sh.P * esz) : up1k(RB * sh.P * 4);
  return 2 * kv + up1k(RB * sh.P * 4) + 4 * (RB * (ks + 4) + 128);
}
void round_layout(const Shape& sh, int n_req, int esz, RoundArgs* a) {
  const int tpr = sh.N / 4;
  const int rows_wg = RT / tpr;
  const bool pow2 = (tpr & (tpr - 1)) == 0;
  const bool many = (int64_t)n_req * sh.nh >= WIDE_MIN_PAIRS;
  const bool wide = many && sh.P >= WIDE_MIN_P;
  int passes = 1;
  const int need = (sh.P + rows_wg - 1) / rows_wg;  // row passes one head takes
  if (wide && pow2) {
    passes = need < WIDE_PASSES ? need : WIDE_PASSES;
  } else if (many && pow2) {
    // the narrow layout over many pairs: tiles of up to MID_PASSES passes, balanced over the head
    const int tiles = (need + MID_PASSES - 1) / MID_PASSES;
    passes = (need + tiles - 1) / tiles;
  }
  a->tile_rows = passes * rows_wg;
  a->n_tiles = (sh.P + a->tile_rows - 1) / a->tile_rows;
  int ks = KS_MIN;
  if (wide) {
    ks = WIDE_KS;
    // no wider than the window needs, and LDS for at least two workgroups per CU
    while (ks > KS_MIN && (ks / 2 >= sh.W || attn_lds(sh, esz, ks) > 80 * 1024)) ks /= 2;
  }
  a->ks = ks;
  a->n_split = (sh.W + ks - 1) / ks + 1;
}
int round_max_splits(const Shape& sh) { return (sh.W + KS_MIN - 1) / KS_MIN + 1; }

static size_t tile_lds_bytes(const Shape& sh, int rw) {
  return (size_t)up1k(RMAXC * sh.N * 4) + up1k(RB * sh.N * 4) + up1k(RMAXC * rw * 4) + up1k(RB * rw * 4) +
         4 * (3 * RMAXC + 4 + RB + RB * RT);
}

size_t round_lds_bytes(const Shape& sh, int esz, const RoundArgs& a) {
  const size_t tile = tile_lds_bytes(sh, a.tile_rows);
  const size_t attn = a.n_split ? (size_t)attn_lds(sh, esz, a.ks) : 0;
  const int ns = a.do_draft ? a.n_split : 0;
  const size_t merge = ns ? (size_t)up1k(ns * RB * 2 * 4) + up1k(ns * RB * 4) + 4 * 256 + up1k(RB * sh.P * 4) : 0;
  size_t m = tile > attn ? tile : attn;
  return m > merge ? m : merge;
}

template <typename T, int G>
static hipError_t launch_round_t(const Shape& sh, const RoundArgs& a, const ReqTable& rt, size_t lds, hipStream_t s) {
  void (*kern)(Shape, RoundArgs, ReqTable);
  if constexpr (G <= MID_PASSES)
    kern = k_round<T, G>;
  else
    kern = k_round_wide<T, G>;
  if (lds > 65536) {
    // Above 64 KiB of dynamic LDS the kernel has to opt in (gfx950 has 160 KiB per workgroup).
    // Done once per process and instantiation with the largest size any shape needs, so later calls
    // (possibly under stream capture) launch only kernels.
    static std::once_flag once;
    static hipError_t set_err = hipSuccess;
    std::call_once(once, [kern] {
      set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                    160 * 1024 - 256);
    });
    if (set_err != hipSuccess) return set_err;
  }
  const int per = a.n_tiles + a.n_split;
  const unsigned items = (unsigned)(rt.n_req * sh.nh * per);
  hipLaunchKernelGGL(kern, dim3((items + 7) / 8 * 8), dim3(RT), lds, s, sh, a, rt);
  return hipGetLastError();
}

// The per-(request, head) kernels take bf16 draft rounds over many pairs with two workgroups per
// CU: the Mamba-2 memory with heads of 48, 64 or 80 dimensions and up to 128 state columns on the
// matrix-core commit; otherwise (gated delta rule, last-W memory, other heads) round_tile's commit
// where its whole head fits one tile (power-of-two threads per row of H, at most WIDE_PASSES passes).
constexpr int PAIR_MAX_LDS = 80 * 1024;
template <int NPC, bool M2, int NBW>
static hipError_t launch_pair_t(const Shape& sh, const RoundArgs& a, const ReqTable& rt, int commit_bytes,
                                size_t lds, hipStream_t s) {
  auto kern = k_round_pair<bf16, NPC, M2, NBW>;
  static std::once_flag once;
  static hipError_t set_err = hipSuccess;
  std::call_once(once, [kern] {
    set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  PAIR_MAX_LDS);
  });
  if (set_err != hipSuccess) return set_err;
  const unsigned items = (unsigned)(rt.n_req * sh.nh);
  hipLaunchKernelGGL(kern, dim3((items + 7) / 8 * 8), dim3(RT), lds, s, sh, a, rt, commit_bytes);
  return hipGetLastError();
}

static hipError_t launch_round_pair(const Shape& sh, const RoundArgs& a0, const ReqTable& rt, hipStream_t s,
                                    bool* taken) {
  *taken = false;
  if (!a0.do_draft || rt.n_req * sh.nh < WIDE_MIN_PAIRS || sh.W < RB) return hipSuccess;
  const int tpr = sh.N / 4, rows_wg = RT / tpr;
  const int npc = sh.P / 16, nb = sh.N / 16;
  const bool m2 = !sh.gdn && !sh.lastw && npc >= 3 && npc <= 5 && nb <= 8;
  RoundArgs a = a0;
  int commit_bytes;
  if (m2) {
    commit_bytes = m2_commit_bytes(sh.P, sh.N);
  } else {
    const int passes = (sh.P + rows_wg - 1) / rows_wg;
    if ((tpr & (tpr - 1)) != 0 || passes > WIDE_PASSES) return hipSuccess;
    a.tile_rows = passes * rows_wg;
    a.n_tiles = 1;
    commit_bytes = (int)tile_lds_bytes(sh, a.tile_rows);
  }
  const PairLds<bf16> L(sh, commit_bytes, m2);
  if (L.total > PAIR_MAX_LDS) return hipSuccess;
  *taken = true;
  a.d_per = Div(1);
  a.d_nh = Div(sh.nh);
  a.d_p4 = Div(sh.P / 4);
  a.d_p = Div(sh.P);
  a.d_tpr = Div(tpr);
  a.d_tr = Div(a.tile_rows > 0 ? a.tile_rows : 1);
  const size_t lds = (size_t)L.total;
  if (!m2) return launch_pair_t<0, false, 1>(sh, a, rt, commit_bytes, lds, s);
  const bool two = nb > 4;
  switch (npc) {
    case 3: return two ? launch_pair_t<3, true, 2>(sh, a, rt, commit_bytes, lds, s)
                       : launch_pair_t<3, true, 1>(sh, a, rt, commit_bytes, lds, s);
    case 4: return two ? launch_pair_t<4, true, 2>(sh, a, rt, commit_bytes, lds, s)
                       : launch_pair_t<4, true, 1>(sh, a, rt, commit_bytes, lds, s);
    default: return two ? launch_pair_t<5, true, 2>(sh, a, rt, commit_bytes, lds, s)
                        : launch_pair_t<5, true, 1>(sh, a, rt, commit_bytes, lds, s);
  }
}

hipError_t launch_round(int dtype, const Shape& sh, const RoundArgs& a0, const ReqTable& rt, hipStream_t s) {
  if (dtype == HYF_BF16) {
    bool taken = false;
    const hipError_t e = launch_round_pair(sh, a0, rt, s, &taken);
    if (taken || e != hipSuccess) return e;
  }
  RoundArgs a = a0;
  a.d_per = Div(a.n_tiles + a.n_split);
  a.d_nh = Div(sh.nh);
  a.d_p4 = Div(sh.P / 4);
  a.d_p = Div(sh.P);
  a.d_tpr = Div(sh.N / 4);
  a.d_tr = Div(a.tile_rows);
  const size_t lds = round_lds_bytes(sh, dtype == HYF_BF16 ? 2 : 4, a);
  if (lds > 160 * 1024 - 256) return hipErrorInvalidValue;
  const int rows_wg = RT / (sh.N / 4);
  const bool wide = a.tile_rows > MID_PASSES * rows_wg;  // tiles of more passes than the narrow kernel keeps
  if (wide && a.tile_rows > WIDE_PASSES * rows_wg) return hipErrorInvalidValue;
  const bool one = a.tile_rows == rows_wg;  // tiles of one pass: the smallest register footprint
  if (dtype == HYF_BF16)
    return wide ? launch_round_t<bf16, WIDE_PASSES>(sh, a, rt, lds, s)
                : one ? launch_round_t<bf16, 1>(sh, a, rt, lds, s) : launch_round_t<bf16, MID_PASSES>(sh, a, rt, lds, s);
  return wide ? launch_round_t<float, WIDE_PASSES>(sh, a, rt, lds, s)
              : one ? launch_round_t<float, 1>(sh, a, rt, lds, s) : launch_round_t<float, MID_PASSES>(sh, a, rt, lds, s);
}

hipError_t launch_ring_append(int dtype, const Shape& sh, char* pool, const ReqTable& rt, const void* k,
                              int64_t ld_k, const void* vT, int64_t ld_v, const float* dtT, int64_t ld_dt,
                              hipStream_t s) {
  const int64_t per = (int64_t)sh.W * sh.P;
  dim3 grid((unsigned)rt.n_req * sh.nh, (unsigned)((per + 255) / 256 < 16 ? (per + 255) / 256 : 16));
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_ring_append<bf16>, grid, dim3(256), 0, s, sh, pool, rt, static_cast<const bf16*>(k), ld_k,
                       static_cast<const bf16*>(vT), ld_v, dtT, ld_dt);
  else
    hipLaunchKernelGGL(k_ring_append<float>, grid, dim3(256), 0, s, sh, pool, rt, static_cast<const float*>(k), ld_k,
                       static_cast<const float*>(vT), ld_v, dtT, ld_dt);
  return hipGetLastError();
}

hipError_t launch_lastw_gather(int dtype, const Shape& sh, char* pool, const ReqTable& rt, void* vb, int64_t ld_vb,
                               float* dtT, int64_t ld_dt, hipStream_t s) {
  const int nblk = (sh.W + HYF_TBLK - 1) / HYF_TBLK;
  dim3 grid((unsigned)(rt.n_req * (sh.nh + sh.G) * nblk));
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_lastw_gather<bf16>, grid, dim3(256), 0, s, sh, pool, rt, static_cast<bf16*>(vb), ld_vb, dtT,
                       ld_dt, nblk);
  else
    hipLaunchKernelGGL(k_lastw_gather<float>, grid, dim3(256), 0, s, sh, pool, rt, static_cast<float*>(vb), ld_vb,
                       dtT, ld_dt, nblk);
  return hipGetLastError();
}

hipError_t launch_bump_counts(char* pool, const Shape& sh, const ReqTable& rt, hipStream_t s) {
  hipLaunchKernelGGL(k_bump_counts, dim3(1), dim3(HYF_MAX_REQUESTS), 0, s, pool, sh, rt);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, uint64_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const uint64_t words = bytes / 4;
  unsigned blocks = (unsigned)((words + 255) / 256 < 2048 ? (words + 255) / 256 : 2048);
  hipLaunchKernelGGL(k_zero, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

hipError_t launch_reset_states(char* pool, const Shape& sh, const ReqTable& rt, hipStream_t s) {
  const uint64_t words = sh.st_bytes / 4;
  unsigned bx = (unsigned)((words + 255) / 256 < 256 ? (words + 255) / 256 : 256);
  hipLaunchKernelGGL(k_reset_states, dim3(bx, rt.n_req), dim3(256), 0, s, pool, sh, rt);
  return hipGetLastError();
}

}  // namespace hyf
