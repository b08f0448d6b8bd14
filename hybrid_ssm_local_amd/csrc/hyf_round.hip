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
  const int prow = t / tpr, c4 = t % tpr;
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
  stage16(nrows * tpr, Bl, [&](int i) { return a.proj + (crow0 + i / tpr) * ld + sh.off_b + grp * N + 4 * (i % tpr); });
  stage4(nrows * trows, xv, [&](int i) { return a.proj + (crow0 + i / trows) * ld + sh.off_v + h * P + tcol(i % trows); });
  if (a.do_draft) {
    stage16(RB * tpr, Cl, [&](int i) { return a.proj + (brow0 + i / tpr) * ld + sh.off_c + grp * N + 4 * (i % tpr); });
    stage4(RB * trows, vb, [&](int i) { return a.proj + (brow0 + i / trows) * ld + sh.off_v + h * P + tcol(i % trows); });
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
    for (int tt = first; tt < nrows; ++tt) {
      const int64_t s = (count + tt) % W;  // uniform
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
  stage16(RB * P4, qs, [&](int i) { return a.proj + (brow0 + i / P4) * ld + sh.off_q + h * P + 4 * (i % P4); });
  const int m = nrows < W ? nrows : W;  // committed rows that land in the ring
  float fk[FIX], fv[FIX];
  if (blk) {
    float* bk = reinterpret_cast<float*>(kst);
    float* bv = reinterpret_cast<float*>(vst);
    stage16(RB * P4, bk, [&](int i) { return a.proj + (brow0 + i / P4) * ld + sh.off_k + h * P + 4 * (i % P4); });
    stage16(RB * P4, bv, [&](int i) { return a.proj + (brow0 + i / P4) * ld + sh.off_v + h * P + 4 * (i % P4); });
  } else {
    const int nslots = W - k0 < ks ? W - k0 : ks;
    const T* K = ring_ptr<T>(a.state_pool, sh, slot, sh.st_k, h) + (int64_t)k0 * P;
    const T* V = ring_ptr<T>(a.state_pool, sh, slot, sh.st_v, h) + (int64_t)k0 * P;
    stage16(nslots * P / VN, kst, [&](int i) { return K + i * VN; });
    stage16(nslots * P / VN, vst, [&](int i) { return V + i * VN; });
#pragma unroll
    for (int e = 0; e < FIX; ++e) {
      const int idx = t + e * RT;
      fk[e] = fv[e] = 0.f;
      if (idx < m * P) {
        const int64_t row = crow0 + nrows - m + idx / P;
        fk[e] = a.proj[row * ld + sh.off_k + h * P + idx % P];
        fv[e] = a.proj[row * ld + sh.off_v + h * P + idx % P];
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
    const int lead = (int)((count + nrows - m) % W);
#pragma unroll
    for (int e = 0; e < FIX; ++e) {
      const int idx = t + e * RT;
      if (idx < m * P) {
        int key = lead + idx / P;
        if (key >= W) key -= W;
        key -= k0;
        if (key >= 0 && key < nk) {
          kst[key * P + idx % P] = from_f32<T>(fk[e]);
          vst[key * P + idx % P] = from_f32<T>(fv[e]);
        }
      }
    }
    __syncthreads();
  }
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
  stage16_dev(RB * P4, memv, [&](int i) { return a.mem + (((int64_t)r * RB + i / P4) * nh + h) * P + 4 * (i % P4); });
  T* out = static_cast<T*>(a.o_in);
  bool first = true;  // uniform: the factors are formed after the first round trip
  for (int e = 0; e < MQ; ++e) {
    if (e * RT >= RB * P4) break;  // uniform
    const int q = t + e * RT;      // this thread's group of 4 outputs: row q / P4, columns 4 (q % P4) ..
    const bool mine = q < RB * P4;
    const int j = mine ? q / P4 : 0;
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
      const int pp = 4 * (q % P4);
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
  const int rh = item / per, role = item % per;
  const int r = rh / nh, h = rh % nh;
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

size_t round_lds_bytes(const Shape& sh, int esz, const RoundArgs& a) {
  const int rw = a.tile_rows;
  const size_t tile = (size_t)up1k(RMAXC * sh.N * 4) + up1k(RB * sh.N * 4) + up1k(RMAXC * rw * 4) + up1k(RB * rw * 4) +
                      4 * (3 * RMAXC + 4 + RB + RB * RT);
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

hipError_t launch_round(int dtype, const Shape& sh, const RoundArgs& a, const ReqTable& rt, hipStream_t s) {
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
