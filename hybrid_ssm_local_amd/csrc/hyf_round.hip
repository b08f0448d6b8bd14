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
// One round in two launches.  k_round: workgroup roles per (request r, head h), in block-index
// order:
//   tiles  [0, n_tiles):   rows p0 .. p0 + rows_wg of H: fold the round's committed rows in (one
//                          read-modify-write), memory readout of the block rows from the updated
//                          rows, and (tile 0) the ring append of the committed (k, v);
//   splits [n_tiles, +n_split): attention of the 8 block rows over 64 ring slots (the last split:
//                          over the block rows themselves), written as (max, sum, output) partials.
// A split sees the ring as it is after this round's append without waiting for it: a slot that
// the append overwrites is read from the projection instead (rounded to the storage dtype, as the
// ring stores it).  k_round_merge then merges the splits per (r, h), adds the readout, writes the
// output projection's input and advances the committed count.  (Merging inside k_round by its
// last workgroup per head needs a device-scope release per workgroup, which on this chip writes
// back the L2 and cost more than the extra launch.)

template <typename T>
__device__ __forceinline__ void round_tile(const Shape& sh, const RoundArgs& a, const ReqTable& rt, int r, int h,
                                           int tile, float* smem) {
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
  float* Bl = smem;                     // [RMAXC][N]  B of the committed rows
  float* Cl = Bl + RMAXC * N;           // [RB][N]     C of the block rows
  float* xv = Cl + RB * N;              // [RMAXC][rows_wg] x (= v) of the committed rows
  float* vb = xv + RMAXC * rows_wg;     // [RB][rows_wg]    v of the block rows
  float* wl = vb + RB * rows_wg;        // [RMAXC] weights, then the total decay
  float* red = wl + RMAXC + 4;          // [RB][RT]

  // every load first (one round trip), then the arithmetic
  float* Hh = h_ptr(a.state_pool, sh, slot, h);
  f32x4 hv = f32x4{0.f, 0.f, 0.f, 0.f};
  if (active) hv = *reinterpret_cast<const f32x4*>(Hh + (int64_t)p * N + 4 * c4);
  for (int idx = t; idx < nrows * tpr; idx += RT) {
    const int tt = idx / tpr, c = idx % tpr;
    *reinterpret_cast<f32x4*>(Bl + tt * N + 4 * c) =
        *reinterpret_cast<const f32x4*>(a.proj + (crow0 + tt) * ld + sh.off_b + grp * N + 4 * c);
  }
  if (a.do_draft)
    for (int idx = t; idx < RB * tpr; idx += RT) {
      const int j = idx / tpr, c = idx % tpr;
      *reinterpret_cast<f32x4*>(Cl + j * N + 4 * c) =
          *reinterpret_cast<const f32x4*>(a.proj + (brow0 + j) * ld + sh.off_c + grp * N + 4 * c);
    }
  for (int idx = t; idx < nrows * rows_wg; idx += RT) {
    const int tt = idx / rows_wg, pp = p0 + idx % rows_wg;
    xv[idx] = pp < P ? a.proj[(crow0 + tt) * ld + sh.off_v + h * P + pp] : 0.f;
  }
  if (a.do_draft)
    for (int idx = t; idx < RB * rows_wg; idx += RT) {
      const int j = idx / rows_wg, pp = p0 + idx % rows_wg;
      vb[idx] = pp < P ? a.proj[(brow0 + j) * ld + sh.off_v + h * P + pp] : 0.f;
    }
  if (t < 64) {
    // weights relative to the last committed row: w_t = dt_t exp(sum_{tau > t} dt_tau A), and
    // the decay exp(sum_t dt_t A) of the old state; lane t < nrows holds row t
    const float raw = t < nrows ? a.proj[(crow0 + t) * ld + sh.off_dt + h] : 0.f;
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
  __syncthreads();

  if (active && nrows > 0) {
    hv *= wl[RMAXC];
    for (int tt = 0; tt < nrows; ++tt) {
      const float xw = xv[tt * rows_wg + prow] * wl[tt];
      const f32x4 b = *reinterpret_cast<const f32x4*>(Bl + tt * N + 4 * c4);
      hv += xw * b;
    }
    *reinterpret_cast<f32x4*>(Hh + (int64_t)p * N + 4 * c4) = hv;
  }

  if (a.do_draft) {
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      float s = 0.f;
      if (active) {
        const f32x4 c = *reinterpret_cast<const f32x4*>(Cl + j * N + 4 * c4);
        s = hv[0] * c[0] + hv[1] * c[1] + hv[2] * c[2] + hv[3] * c[3];
      }
      red[j * RT + t] = s;
    }
    __syncthreads();
    const float D = a.d_skip[h];
    for (int idx = t; idx < RB * rows_wg; idx += RT) {
      const int j = idx / rows_wg, pr = idx % rows_wg;
      const int pp = p0 + pr;
      if (pp >= P) continue;
      float s = 0.f;
      for (int c = 0; c < tpr; ++c) s += red[j * RT + pr * tpr + c];
      a.mem[(((int64_t)r * RB + j) * nh + h) * P + pp] = s + D * vb[idx];
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

template <typename T>
__device__ __forceinline__ void round_attn(const Shape& sh, const RoundArgs& a, const ReqTable& rt, int r, int h,
                                           int sp, float* smem) {
  constexpr int VN = Vec16<T>::n;
  typedef typename Vec16<T>::type Vv;
  const int nh = sh.nh, P = sh.P, W = sh.W;
  const int PK = P + 1;  // key rows padded so consecutive keys fall in different banks
  float* qs = smem;                   // [RB][P]
  float* ks = qs + RB * P;            // [ATT_KS][P + 1]
  float* vs = ks + ATT_KS * PK;       // [ATT_KS][P]
  float* pl = vs + ATT_KS * P;        // [RB][ATT_KS]
  const int slot = rt.slot[r];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t ld = a.ld;
  const int64_t brow0 = a.blk_row0 + (int64_t)r * RB;
  const bool blk = sp == a.n_split - 1;
  const int nrows = a.do_commit ? rt.row0[r + 1] - rt.row0[r] : 0;
  const int64_t crow0 = rt.row0[r];

  const float scale = rsqrtf((float)P);
  for (int idx = t; idx < RB * P / 4; idx += RT) {
    const int j = 4 * idx / P, pp = 4 * idx % P;
    *reinterpret_cast<f32x4*>(qs + j * P + pp) =
        *reinterpret_cast<const f32x4*>(a.proj + (brow0 + j) * ld + sh.off_q + h * P + pp) * scale;
  }
  int nk;
  if (blk) {
    nk = RB;
    for (int idx = t; idx < RB * P / 4; idx += RT) {
      const int j = 4 * idx / P, pp = 4 * idx % P;
      const f32x4 kk = *reinterpret_cast<const f32x4*>(a.proj + (brow0 + j) * ld + sh.off_k + h * P + pp);
      const f32x4 vv = *reinterpret_cast<const f32x4*>(a.proj + (brow0 + j) * ld + sh.off_v + h * P + pp);
#pragma unroll
      for (int e = 0; e < 4; ++e) ks[j * PK + pp + e] = kk[e];
      *reinterpret_cast<f32x4*>(vs + j * P + pp) = vv;
    }
  } else {
    // ring slots k0 .. k0 + nk - 1 of the window after this round's append
    const int64_t count = *count_ptr(a.state_pool, sh, slot);
    const int64_t tot = count + nrows;
    const int valid = (int)(tot < W ? tot : W);
    const int k0 = sp * ATT_KS;
    nk = valid - k0;
    nk = nk < 0 ? 0 : (nk > ATT_KS ? ATT_KS : nk);
    const int m = nrows < W ? nrows : W;             // rows of this round that land in the ring
    const int lead = (int)((count + nrows - m) % W);  // slot of the first of them
    const T* K = ring_ptr<T>(a.state_pool, sh, slot, sh.st_k, h);
    const T* V = ring_ptr<T>(a.state_pool, sh, slot, sh.st_v, h);
    const int CH = P / VN;  // 16-byte chunks per key row
    for (int idx = t; idx < nk * CH; idx += RT) {
      const int key = idx / CH, c = idx % CH;
      const int s = k0 + key;
      const int jn = (s - lead + W) % W;  // index among the landing rows, if this slot is one
      float kf[VN], vf[VN];
      if (jn < m) {
        const int64_t row = crow0 + (nrows - m) + jn;
#pragma unroll
        for (int e = 0; e < VN; ++e) {
          kf[e] = to_f32(from_f32<T>(a.proj[row * ld + sh.off_k + h * P + c * VN + e]));
          vf[e] = to_f32(from_f32<T>(a.proj[row * ld + sh.off_v + h * P + c * VN + e]));
        }
      } else {
        const Vv kv = *reinterpret_cast<const Vv*>(K + (int64_t)s * P + c * VN);
        const Vv vv = *reinterpret_cast<const Vv*>(V + (int64_t)s * P + c * VN);
#pragma unroll
        for (int e = 0; e < VN; ++e) {
          kf[e] = to_f32(kv[e]);
          vf[e] = to_f32(vv[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        ks[key * PK + c * VN + e] = kf[e];
        vs[key * P + c * VN + e] = vf[e];
      }
    }
  }
  float* op = a.att_part + ((((int64_t)r * nh + h) * a.n_split + sp) * RB) * P;
  float* ml = a.att_ml + ((((int64_t)r * nh + h) * a.n_split + sp) * RB) * 2;
  if (nk == 0) {
    for (int idx = t; idx < RB * P; idx += RT) op[idx] = 0.f;
    if (t < RB) {
      ml[2 * t] = -INFINITY;
      ml[2 * t + 1] = 0.f;
    }
    return;
  }
  __syncthreads();

  // scores: lane = key, wave w handles block rows w and w + 4
  const int key = lane;
  float sc[2];
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int j = wave + 4 * q2;
    float acc = 0.f;
    if (key < nk)
      for (int pp = 0; pp < P; ++pp) acc += qs[j * P + pp] * ks[key * PK + pp];
    bool ok = key < nk;
    if (blk && !sh.cross && key != j) ok = false;
    sc[q2] = ok ? acc : -INFINITY;
  }
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int j = wave + 4 * q2;
    const float mx = wave_max(sc[q2]);
    const float e = sc[q2] == -INFINITY ? 0.f : expf(sc[q2] - mx);
    const float l = wave_sum(e);
    pl[j * ATT_KS + key] = e;
    if (lane == 0) {
      ml[2 * j] = mx;
      ml[2 * j + 1] = l;
    }
  }
  __syncthreads();
  for (int idx = t; idx < RB * P; idx += RT) {
    const int j = idx / P, pp = idx % P;
    float acc = 0.f;
    for (int k2 = 0; k2 < nk; ++k2) acc += pl[j * ATT_KS + k2] * vs[k2 * P + pp];
    op[idx] = acc;
  }
}

template <typename T>
__device__ __forceinline__ void round_merge(const Shape& sh, const RoundArgs& a, int r, int h, float* smem) {
  const int nh = sh.nh, P = sh.P, t = threadIdx.x;
  const int ns = a.n_split;
  const float* ml = a.att_ml + (((int64_t)r * nh + h) * ns) * RB * 2;
  const float* op = a.att_part + (((int64_t)r * nh + h) * ns) * RB * P;
  float* sml = smem;  // [ns][RB][2]
  for (int idx = t; idx < ns * RB * 2; idx += RT) sml[idx] = ml[idx];
  __syncthreads();
  T* out = static_cast<T*>(a.o_in);
  for (int idx = t; idx < RB * P; idx += RT) {
    const int j = idx / P, pp = idx % P;
    float m = -INFINITY;
    for (int s = 0; s < ns; ++s) m = fmaxf(m, sml[(s * RB + j) * 2]);
    float l = 0.f, o = 0.f;
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
      const float ms = sml[(s * RB + j) * 2];
      const float f = ms == -INFINITY ? 0.f : expf(ms - m);
      l += f * sml[(s * RB + j) * 2 + 1];
      o += f * op[((int64_t)s * RB + j) * P + pp];
    }
    const float mem = a.mem[(((int64_t)r * RB + j) * nh + h) * P + pp];
    out[((int64_t)r * RB + j) * sh.dq + h * P + pp] = from_f32<T>(o / l + mem);
  }
}

template <typename T>
__global__ void __launch_bounds__(RT) k_round(Shape sh, RoundArgs a, ReqTable rt) {
  extern __shared__ __attribute__((aligned(16))) float dsm[];
  const int per = a.n_tiles + a.n_split;
  const int rh = blockIdx.x / per, role = blockIdx.x % per;
  const int r = rh / sh.nh, h = rh % sh.nh;
  if (role < a.n_tiles)
    round_tile<T>(sh, a, rt, r, h, role, dsm);
  else
    round_attn<T>(sh, a, rt, r, h, role - a.n_tiles, dsm);
}

// Per (request, head): merge the attention splits, add the readout, write the output
// projection's input; head 0 then advances the request's committed count (every reader of the
// count ran in the previous launch).
template <typename T>
__global__ void __launch_bounds__(RT) k_round_merge(Shape sh, RoundArgs a, ReqTable rt) {
  extern __shared__ __attribute__((aligned(16))) float dsm[];
  const int r = blockIdx.x / sh.nh, h = blockIdx.x % sh.nh;
  round_merge<T>(sh, a, r, h, dsm);
  if (h == 0 && threadIdx.x == 0 && a.do_commit)
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

size_t round_lds_bytes(const Shape& sh, int n_split) {
  const size_t rw = round_rows_per_tile(sh);
  const size_t tile = sizeof(float) * ((size_t)(RMAXC + RB) * sh.N + (RMAXC + RB) * rw + RMAXC + 4 + RB * RT);
  const size_t attn = sizeof(float) * ((size_t)RB * sh.P + (size_t)ATT_KS * (sh.P + 1) + (size_t)ATT_KS * sh.P + RB * ATT_KS);
  const size_t merge = sizeof(float) * (size_t)n_split * RB * 2;
  size_t m = tile > attn ? tile : attn;
  return m > merge ? m : merge;
}

hipError_t launch_round(int dtype, const Shape& sh, const RoundArgs& a, const ReqTable& rt, hipStream_t s) {
  const int per = a.n_tiles + a.n_split;
  const size_t lds = round_lds_bytes(sh, a.n_split);
  if (lds > 65536) {
    // Above 64 KiB of dynamic LDS the kernel has to opt in (gfx950 has 160 KiB per workgroup).
    // Done once per process with the largest size any shape needs, so later calls (possibly under
    // stream capture) launch only kernels.
    static std::once_flag once;
    static hipError_t set_err = hipSuccess;
    std::call_once(once, [] {
      const int mx = 160 * 1024;
      const void* fns[4] = {reinterpret_cast<const void*>(k_round<bf16>), reinterpret_cast<const void*>(k_round<float>),
                            reinterpret_cast<const void*>(k_round_merge<bf16>),
                            reinterpret_cast<const void*>(k_round_merge<float>)};
      for (const void* f : fns)
        if (set_err == hipSuccess) set_err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, mx);
    });
    if (set_err != hipSuccess) return set_err;
  }
  dim3 grid((unsigned)(rt.n_req * sh.nh * per));
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_round<bf16>, grid, dim3(RT), lds, s, sh, a, rt);
  else
    hipLaunchKernelGGL(k_round<float>, grid, dim3(RT), lds, s, sh, a, rt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.do_draft) return a.do_commit ? launch_bump_counts(a.state_pool, sh, rt, s) : hipSuccess;
  const size_t mlds = sizeof(float) * (size_t)a.n_split * RB * 2;
  dim3 mgrid((unsigned)(rt.n_req * sh.nh));
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_round_merge<bf16>, mgrid, dim3(RT), mlds, s, sh, a, rt);
  else
    hipLaunchKernelGGL(k_round_merge<float>, mgrid, dim3(RT), mlds, s, sh, a, rt);
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
