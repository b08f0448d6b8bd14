// Kernels of one draft/commit round (k_round, see below) and the ring/state helpers of a prefill
// commit (k_ring_append, k_bump_counts, k_reset_states, k_zero).
#include <mutex>

#include "hyf_launch.h"

namespace hyf {

constexpr int RB = HYF_BLOCK;   // block rows
constexpr int RMAXC = 16;       // largest per-request commit a round kernel folds in
constexpr int ATT_KS = 64;      // keys per attention split
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

// ---------------------------------------------------------------------------------------------
// One round, one launch.  Workgroup roles per (request r, head h), in block-index order:
//   tiles  [0, n_tiles):   rows p0 .. p0 + rows_wg of H: fold the round's committed rows in (one
//                          read-modify-write), memory readout of the block rows from the updated
//                          rows, and (tile 0) the ring append of the committed (k, v);
//   splits [n_tiles, +n_split): attention of the 8 block rows over 64 ring slots (the last split:
//                          over the block rows themselves), written as (max, sum, output) partials.
// A split sees the ring as it is after this round's append without waiting for it: a slot that
// the append overwrites is read from the projection instead (rounded to the storage dtype, as the
// ring stores it).  The last workgroup of (r, h) to finish (a counter) merges the splits, adds the
// readout and writes the output projection's input; the last head of a request advances the
// request's committed count.  The counters are cleared by the round's input projection.

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
// x (= v) of the committed rows [RMAXC][rows_wg] f32 | v of the block rows [RB][rows_wg] f32 |
// weights [RMAXC + 4] (gated delta rule: retention gates) | write gates [RMAXC] | inverse key norms
// [RMAXC] | inverse query norms [RB] | readout partials [RB][RT].
//
// Gated delta-rule memory (sh.gdn): the committed rows are folded one at a time, each row of H
// (tpr threads) forming H_p . k with a reduction over its threads, then
// H_p <- alpha (H_p - beta (H_p . k) k) + beta x_p k, k the unit-normalized B row; the readout
// uses the unit-normalized C rows.
template <typename T>
__device__ __forceinline__ void round_tile(const Shape& sh, const RoundArgs& a, const ReqTable& rt, int r, int h,
                                           int tile, char* smem) {
  const int nh = sh.nh, P = sh.P, N = sh.N;
  const int tpr = N / 4;           // threads per H row (4 columns each)
  const int rows_wg = RT / tpr;    // H rows per tile
  const int t = threadIdx.x;
  const int prow = t / tpr, c4 = t % tpr;
  const int p0 = tile * rows_wg, p = p0 + prow;
  const bool active = prow < rows_wg && p < P;
  const int slot = rt.slot[r];
  const int grp = h / (nh / sh.G);
  const int nrows = a.do_commit ? rt.row0[r + 1] - rt.row0[r] : 0;
  const int64_t crow0 = rt.row0[r];
  const int64_t brow0 = a.blk_row0 + (int64_t)r * RB;
  const int64_t ld = a.ld;
  float* Bl = reinterpret_cast<float*>(smem);
  float* Cl = reinterpret_cast<float*>(smem + up1k(RMAXC * N * 4));
  float* xv = reinterpret_cast<float*>(reinterpret_cast<char*>(Cl) + up1k(RB * N * 4));
  float* vb = reinterpret_cast<float*>(reinterpret_cast<char*>(xv) + up1k(RMAXC * rows_wg * 4));
  float* wl = reinterpret_cast<float*>(reinterpret_cast<char*>(vb) + up1k(RB * rows_wg * 4));
  float* ga = wl + RMAXC + 4;  // write gates (gated delta rule)
  float* ik = ga + RMAXC;      // inverse key norms
  float* iq = ik + RMAXC;      // inverse query norms
  float* red = iq + RB;

  // every load first (one round trip), then the arithmetic
  float* Hh = h_ptr(a.state_pool, sh, slot, h);
  f32x4 hv = f32x4{0.f, 0.f, 0.f, 0.f};
  if (active) hv = *reinterpret_cast<const f32x4*>(Hh + (int64_t)p * N + 4 * c4);
  const float raw = t < nrows ? a.proj[(crow0 + t) * ld + sh.off_dt + h] : 0.f;
  const float rawb = sh.gdn && t < nrows ? a.proj[(crow0 + t) * ld + sh.off_beta + h] : 0.f;
  stage16(nrows * tpr, Bl, [&](int i) { return a.proj + (crow0 + i / tpr) * ld + sh.off_b + grp * N + 4 * (i % tpr); });
  stage4(nrows * rows_wg, xv, [&](int i) { return a.proj + (crow0 + i / rows_wg) * ld + sh.off_v + h * P + p0 + i % rows_wg; });
  if (a.do_draft) {
    stage16(RB * tpr, Cl, [&](int i) { return a.proj + (brow0 + i / tpr) * ld + sh.off_c + grp * N + 4 * (i % tpr); });
    stage4(RB * rows_wg, vb, [&](int i) { return a.proj + (brow0 + i / rows_wg) * ld + sh.off_v + h * P + p0 + i % rows_wg; });
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
        float d = hv[0] * k[0] + hv[1] * k[1] + hv[2] * k[2] + hv[3] * k[3];
        if (pow2) {
          for (int o = tpr / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
        } else {
          red[t] = d;
          __syncthreads();
          d = 0.f;
          for (int c = 0; c < tpr; ++c) d += red[prow * tpr + c];
          __syncthreads();
        }
        const float be = ga[tt];
        const float xw = active ? be * xv[tt * rows_wg + prow] : 0.f;
        hv = wl[tt] * (hv - (be * d) * k) + xw * k;
      }
      if (active) *reinterpret_cast<f32x4*>(Hh + (int64_t)p * N + 4 * c4) = hv;
    }
  } else if (active && nrows > 0) {
    hv *= wl[RMAXC];
    for (int tt = 0; tt < nrows; ++tt) {
      const float xw = xv[tt * rows_wg + prow] * wl[tt];
      const f32x4 b = *reinterpret_cast<const f32x4*>(Bl + tt * N + 4 * c4);
      hv += xw * b;
    }
    *reinterpret_cast<f32x4*>(Hh + (int64_t)p * N + 4 * c4) = hv;
  }

  if (a.do_draft) {
    float sum[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      sum[j] = 0.f;
      if (active) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(Cl + j * N + 4 * c4);
        sum[j] = hv[0] * c[0] + hv[1] * c[1] + hv[2] * c[2] + hv[3] * c[3];
      }
    }
    const float D = a.d_skip[h];
    if (pow2) {
      // the tpr threads of a row are consecutive lanes of one wave: xor-shuffle reduction
      for (int o = tpr / 2; o >= 1; o >>= 1)
#pragma unroll
        for (int j = 0; j < RB; ++j) sum[j] += __shfl_xor(sum[j], o, 64);
      if (active && c4 == 0)
#pragma unroll
        for (int j = 0; j < RB; ++j)
          st_dev(a.mem + (((int64_t)r * RB + j) * nh + h) * P + p,
                 sum[j] * (sh.gdn ? iq[j] : 1.f) + D * vb[j * rows_wg + prow]);
    } else {
#pragma unroll
      for (int j = 0; j < RB; ++j) red[j * RT + t] = sum[j];
      __syncthreads();
      for (int idx = t; idx < RB * rows_wg; idx += RT) {
        const int j = idx / rows_wg, pr = idx % rows_wg;
        const int pp = p0 + pr;
        if (pp >= P) continue;
        float acc = 0.f;
        for (int c = 0; c < tpr; ++c) acc += red[j * RT + pr * tpr + c];
        st_dev(a.mem + (((int64_t)r * RB + j) * nh + h) * P + pp, acc * (sh.gdn ? iq[j] : 1.f) + D * vb[idx]);
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
    for (int idx = t; idx < (nrows - first) * P; idx += RT) {
      const int tt = first + idx / P, pp = idx % P;
      const int64_t s = (count + tt) % W;
      K[s * P + pp] = from_f32<T>(a.proj[(crow0 + tt) * ld + sh.off_k + h * P + pp]);
      V[s * P + pp] = from_f32<T>(a.proj[(crow0 + tt) * ld + sh.off_v + h * P + pp]);
    }
  }
}

// Four consecutive elements (8-byte aligned for bf16, 16-byte for fp32) as fp32.
__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4f(const bf16* p) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]), static_cast<float>(v[3])};
}

// Scores and outputs of one split on fp32 MFMAs (16x16x4): keys from K (row stride P, up to 64
// rows), values from V, queries qs [RB][P] f32.  Wave w computes S^T for keys 16 w .. 16 w + 15
// against the 8 queries (padded to 16 columns); lane (li, lg) supplies, for instruction j of a
// group of four, dimension p0 + 4 lg + j of key 16 w + li and of query li, so one 4-element load
// of each operand feeds four instructions.  Softmax over the 64 keys meets in LDS; the
// probabilities go to LDS and a second set of MFMAs forms P . V with wave w on the 16-column
// tiles w, w + 4, ... of the output.  Keys at or past nk are masked (their rows may hold
// anything: their scores are discarded and their values are multiplied by nothing).
template <typename KT>
__device__ __forceinline__ void attn_split(const Shape& sh, int nk, bool blk, const float* qs, const KT* K,
                                           const KT* V, float* pl, float* red, float* op, float* ml) {
  const int P = sh.P, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const float scale = rsqrtf((float)P);
  // ---- scores S^T[key][q]
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  const int krow = 16 * wave + li;
  if (16 * wave < nk) {
#pragma unroll 4
    for (int p0 = 0; p0 < P; p0 += 16) {
      const f32x4 kv = ld4f(K + krow * P + p0 + 4 * lg);
      f32x4 qv = *reinterpret_cast<const f32x4*>(qs + li * P + p0 + 4 * lg);  // rows >= RB: masked
      if (li >= RB) qv = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) s = Mfma16<float>::mma(kv[j], qv[j], s);
    }
  }
  // lane (li, lg) register rr: key 16 w + 4 lg + rr, query li
  float e[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int key = 16 * wave + 4 * lg + rr;
    bool ok = key < nk && li < RB;
    if (blk && !sh.cross && key != li) ok = false;
    e[rr] = ok ? s[rr] * scale : -INFINITY;
    mloc = fmaxf(mloc, e[rr]);
  }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
  if (lg == 0) red[wave * 16 + li] = mloc;
  __syncthreads();
  float m = -INFINITY;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) m = fmaxf(m, red[w2 * 16 + li]);
  float lsum = 0.f;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    e[rr] = e[rr] == -INFINITY ? 0.f : expf(e[rr] - m);
    lsum += e[rr];
    pl[li * ATT_KS + 16 * wave + 4 * lg + rr] = e[rr];
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (lg == 0) red[64 + wave * 16 + li] = lsum;
  __syncthreads();
  if (wave == 0 && lg == 0 && li < RB) {
    st_dev(ml + 2 * li, m);
    st_dev(ml + 2 * li + 1, red[64 + li] + red[64 + 16 + li] + red[64 + 32 + li] + red[64 + 48 + li]);
  }
  // ---- O[q][p] = sum_key pl[q][key] V[key][p]
  const int nks = (nk + 3) / 4 * 4;
  for (int pt = wave; pt * 16 < P; pt += 4) {
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int k0 = 0; k0 < nks; k0 += 16) {
      const f32x4 pa = *reinterpret_cast<const f32x4*>(pl + li * ATT_KS + k0 + 4 * lg);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + 4 * lg + j;
        const float vv = key < nk ? to_f32(V[key * P + pt * 16 + li]) : 0.f;
        o = Mfma16<float>::mma(pa[j], vv, o);
      }
    }
    // lane (li, lg) register rr: query 4 lg + rr, column pt * 16 + li
    if (lg < 2)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) st_dev(op + (4 * lg + rr) * P + pt * 16 + li, o[rr]);
  }
}

// Attention LDS (bytes): ring K, V of the split [ATT_KS][P] storage dtype | q [RB][P] f32 |
// k, v of the round's committed rows (or of the block rows) [RB][P] f32 each | probabilities
// [16][ATT_KS] | softmax scratch [128].
template <typename T>
__device__ __forceinline__ void round_attn(const Shape& sh, const RoundArgs& a, const ReqTable& rt, int r, int h,
                                           int sp, char* smem) {
  constexpr int VN = Vec16<T>::n;
  const int nh = sh.nh, P = sh.P, W = sh.W;
  T* kst = reinterpret_cast<T*>(smem);
  T* vst = reinterpret_cast<T*>(smem + up1k(ATT_KS * P * (int)sizeof(T)));
  float* qs = reinterpret_cast<float*>(reinterpret_cast<char*>(vst) + up1k(ATT_KS * P * (int)sizeof(T)));
  float* nkf = reinterpret_cast<float*>(reinterpret_cast<char*>(qs) + up1k(RB * P * 4));
  float* nvf = reinterpret_cast<float*>(reinterpret_cast<char*>(nkf) + up1k(RB * P * 4));
  float* pl = reinterpret_cast<float*>(reinterpret_cast<char*>(nvf) + up1k(RB * P * 4));
  float* red = pl + 16 * ATT_KS;
  __shared__ int64_t s_count;
  const int slot = rt.slot[r];
  const int t = threadIdx.x;
  const int64_t ld = a.ld;
  const int64_t brow0 = a.blk_row0 + (int64_t)r * RB;
  const bool blk = sp == a.n_split - 1;
  const int nrows = a.do_commit ? rt.row0[r + 1] - rt.row0[r] : 0;
  const int64_t crow0 = rt.row0[r];
  const int k0 = sp * ATT_KS;
  const int P4 = P / 4;

  // Every load is independent of the committed count, so all go out together: the count, q, the
  // split's ring slots (always inside the ring), and the k, v of the round's committed rows (they
  // replace the slots this round's append overwrites) or of the block rows.
  if (!blk && t == 0) s_count = *count_ptr(a.state_pool, sh, slot);
  stage16(RB * P4, qs, [&](int i) { return a.proj + (brow0 + i / P4) * ld + sh.off_q + h * P + 4 * (i % P4); });
  if (blk) {
    stage16(RB * P4, nkf, [&](int i) { return a.proj + (brow0 + i / P4) * ld + sh.off_k + h * P + 4 * (i % P4); });
    stage16(RB * P4, nvf, [&](int i) { return a.proj + (brow0 + i / P4) * ld + sh.off_v + h * P + 4 * (i % P4); });
  } else {
    const int nslots = W - k0 < ATT_KS ? W - k0 : ATT_KS;
    const T* K = ring_ptr<T>(a.state_pool, sh, slot, sh.st_k, h) + (int64_t)k0 * P;
    const T* V = ring_ptr<T>(a.state_pool, sh, slot, sh.st_v, h) + (int64_t)k0 * P;
    stage16(nslots * P / VN, kst, [&](int i) { return K + i * VN; });
    stage16(nslots * P / VN, vst, [&](int i) { return V + i * VN; });
    stage16(nrows * P4, nkf, [&](int i) { return a.proj + (crow0 + i / P4) * ld + sh.off_k + h * P + 4 * (i % P4); });
    stage16(nrows * P4, nvf, [&](int i) { return a.proj + (crow0 + i / P4) * ld + sh.off_v + h * P + 4 * (i % P4); });
  }
  vm_wait<0>();
  __syncthreads();

  float* op = a.att_part + ((((int64_t)r * nh + h) * a.n_split + sp) * RB) * P;
  float* ml = a.att_ml + ((((int64_t)r * nh + h) * a.n_split + sp) * RB) * 2;
  if (blk) {
    attn_split(sh, RB, true, qs, nkf, nvf, pl, red, op, ml);
    return;
  }
  const int64_t count = s_count;
  const int64_t tot = count + nrows;
  const int valid = (int)(tot < W ? tot : W);
  int nk = valid - k0;
  nk = nk < 0 ? 0 : (nk > ATT_KS ? ATT_KS : nk);
  if (nk == 0) {
    for (int idx = t; idx < RB * P; idx += RT) st_dev(op + idx, 0.f);
    if (t < RB) {
      st_dev(ml + 2 * t, -INFINITY);
      st_dev(ml + 2 * t + 1, 0.f);
    }
    return;
  }
  if (nrows > 0) {
    // the slots this round's append overwrites take its rows, rounded as the ring stores them:
    // slot (count + j) mod W holds row j for the last m = min(nrows, W) rows
    const int m = nrows < W ? nrows : W;
    const int lead = (int)((count + nrows - m) % W);
    for (int idx = t; idx < m * P; idx += RT) {
      const int jn = idx / P, pp = idx % P;
      const int key = (lead + jn) % W - k0;
      if (key >= 0 && key < nk) {
        kst[key * P + pp] = from_f32<T>(nkf[(nrows - m + jn) * P + pp]);
        vst[key * P + pp] = from_f32<T>(nvf[(nrows - m + jn) * P + pp]);
      }
    }
    __syncthreads();
  }
  attn_split(sh, nk, false, qs, kst, vst, pl, red, op, ml);
}

// Merge of one (request, head): the partials of MCH splits at a time are staged in LDS together
// with the (max, sum) pairs and the readout (one round trip); per (split, row) factors
// exp(max_s - max) are formed once, in parallel, then every output sums its splits.
// Merge LDS (bytes): (max, sum) [ns][RB][2] | factors [ns][RB] | row maxima and sums [2 RB] |
// readout [RB][P] | partials [min(MCH, ns)][RB][P] (sized for the splits there are: with 9 splits
// the kernel's LDS stays at the attention's 34 KiB, four workgroups per CU instead of three).
constexpr int MCH = 16;
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
  float* sop = reinterpret_cast<float*>(reinterpret_cast<char*>(memv) + up1k(RB * P * 4));
  constexpr int EPT = 8;  // outputs per thread: RB * P <= 8 * RT for P <= 256
  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
  stage16_dev(ns * RB * 2 / 4, sml, [&](int i) { return ml + 4 * i; });
  stage16_dev(RB * P4, memv, [&](int i) { return a.mem + (((int64_t)r * RB + i / P4) * nh + h) * P + 4 * (i % P4); });
  for (int s0 = 0; s0 < ns; s0 += MCH) {
    const int nc = ns - s0 < MCH ? ns - s0 : MCH;
    stage16_dev(nc * RB * P4, sop, [&](int i) { return op + (int64_t)s0 * RB * P + 4 * i; });
    vm_wait<0>();
    __syncthreads();
    if (s0 == 0) {
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
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int idx = t + e * RT;
      if (idx >= RB * P) continue;
      const int j = idx / P;
      float sum = 0.f;
#pragma unroll 4
      for (int s = 0; s < nc; ++s) sum += fac[(s0 + s) * RB + j] * sop[s * RB * P + idx];
      acc[e] += sum;
    }
    __syncthreads();  // sop is refilled by the next chunk; rowm sums are complete
  }
  T* out = static_cast<T*>(a.o_in);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int idx = t + e * RT;
    if (idx >= RB * P) continue;
    const int j = idx / P, pp = idx % P;
    out[((int64_t)r * RB + j) * sh.dq + h * P + pp] = from_f32<T>(acc[e] / rowm[RB + j] + memv[idx]);
  }
}

template <typename T>
__global__ void __launch_bounds__(RT) k_round(Shape sh, RoundArgs a, ReqTable rt) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  __shared__ int s_last;
  const int nh = sh.nh;
  const int per = a.n_tiles + a.n_split;
  const int rh = blockIdx.x / per, role = blockIdx.x % per;
  const int r = rh / nh, h = rh % nh;
  if (role < a.n_tiles)
    round_tile<T>(sh, a, rt, r, h, role, dsm);
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
    *count_ptr(a.state_pool, sh, rt.slot[r]) += rt.row0[r + 1] - rt.row0[r];
}

template <typename T>
__global__ void __launch_bounds__(256) k_ring_append(Shape sh, char* pool, ReqTable rt, const T* __restrict__ k,
                                                     int64_t ld_k, const T* __restrict__ vT, int64_t ld_v) {
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

// Rows of H per commit tile and tiles per head.
int round_rows_per_tile(const Shape& sh) { return RT / (sh.N / 4); }
int round_tiles(const Shape& sh) { return (sh.P + round_rows_per_tile(sh) - 1) / round_rows_per_tile(sh); }

size_t round_lds_bytes(const Shape& sh, int esz, int n_split) {
  const int rw = round_rows_per_tile(sh);
  const size_t tile = (size_t)up1k(RMAXC * sh.N * 4) + up1k(RB * sh.N * 4) + up1k(RMAXC * rw * 4) + up1k(RB * rw * 4) +
                      4 * (3 * RMAXC + 4 + RB + RB * RT);
  const size_t attn = (size_t)2 * up1k(ATT_KS * sh.P * esz) + 3 * up1k(RB * sh.P * 4) + 4 * (16 * ATT_KS + 128);
  const size_t merge = n_split ? (size_t)up1k(n_split * RB * 2 * 4) + up1k(n_split * RB * 4) + 4 * 256 +
                                     up1k(RB * sh.P * 4) + up1k((n_split < MCH ? n_split : MCH) * RB * sh.P * 4)
                               : 0;
  size_t m = tile > attn ? tile : attn;
  return m > merge ? m : merge;
}

hipError_t launch_round(int dtype, const Shape& sh, const RoundArgs& a, const ReqTable& rt, hipStream_t s) {
  const int per = a.n_tiles + a.n_split;
  const size_t lds = round_lds_bytes(sh, dtype == HYF_BF16 ? 2 : 4, a.do_draft ? a.n_split : 0);
  if (lds > 65536) {
    // Above 64 KiB of dynamic LDS the kernel has to opt in (gfx950 has 160 KiB per workgroup).
    // Done once per process with the largest size any shape needs, so later calls (possibly under
    // stream capture) launch only kernels.
    static std::once_flag once;
    static hipError_t set_err = hipSuccess;
    std::call_once(once, [] {
      const int mx = 160 * 1024 - 256;  // leaves room for the kernel's few bytes of static LDS
      set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_round<bf16>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, mx);
      if (set_err == hipSuccess)
        set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_round<float>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, mx);
    });
    if (set_err != hipSuccess) return set_err;
  }
  dim3 grid((unsigned)(rt.n_req * sh.nh * per));
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_round<bf16>, grid, dim3(RT), lds, s, sh, a, rt);
  else
    hipLaunchKernelGGL(k_round<float>, grid, dim3(RT), lds, s, sh, a, rt);
  return hipGetLastError();
}

hipError_t launch_ring_append(int dtype, const Shape& sh, char* pool, const ReqTable& rt, const void* k,
                              int64_t ld_k, const void* vT, int64_t ld_v, hipStream_t s) {
  const int64_t per = (int64_t)sh.W * sh.P;
  dim3 grid((unsigned)rt.n_req * sh.nh, (unsigned)((per + 255) / 256 < 16 ? (per + 255) / 256 : 16));
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_ring_append<bf16>, grid, dim3(256), 0, s, sh, pool, rt, static_cast<const bf16*>(k), ld_k,
                       static_cast<const bf16*>(vT), ld_v);
  else
    hipLaunchKernelGGL(k_ring_append<float>, grid, dim3(256), 0, s, sh, pool, rt, static_cast<const float*>(k), ld_k,
                       static_cast<const float*>(vT), ld_v);
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
