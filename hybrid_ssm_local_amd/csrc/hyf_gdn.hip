// Gated delta-rule memory: commit of whole prefixes.
//
// Rule per head (one row of H per value feature p, one column per key feature n):
//   H <- alpha_t H (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  k_t = B_t / sqrt(|B_t|^2 + 1e-6),
// with the retention gate alpha_t = sigmoid(raw_alpha + dt_bias[h]) and the write gate
// beta_t = sigmoid(raw_beta + a_log[h]).  The operands come time-blocked from the prefill GEMM:
// x (= v) and B tiled (tile_off), the raw gates plain in a.dt (alpha at feature h, beta at nh + h).
#include <mutex>

#include "hyf_launch.h"

namespace hyf {

constexpr int TB = HYF_TBLK;  // tokens per block of the time-blocked layout

// Gated delta-rule commit of a whole prefix, one token at a time (the rule is not a weighted sum of
// independent writes, so the split over time the Mamba-2 scan uses does not apply): per (request,
// head, block of GDN_ROWS rows of H), 16 threads per row with N / 16 columns each keep the row in
// registers; per block of TB tokens the rows' x, the keys B (token-major, fp32) and the gates come
// to LDS, then for each token the row's H_p . k is a 16-lane shuffle reduction and
// H_p <- alpha (H_p - beta (H_p . k) k) + beta x_p k with k = B / sqrt(|B|^2 + 1e-6).
// Gates: alpha = sigmoid(raw + dt_bias[h]), beta = sigmoid(raw' + a_log[h]) with the raw gates
// time-blocked in a.dt (alpha at feature h, beta at feature nh + h).
constexpr int GDN_ROWS = 16;  // H rows per workgroup: many workgroups, so the whole chip shares the sequential work
// Sum over the 16 lanes of a DPP row (lanes 16 i .. 16 i + 15), every lane getting the total: swaps
// inside quads ([1,0,3,2], then [2,3,0,1]), then the mirrored half-row and the mirrored row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}

template <typename T, int NCH>
__global__ void __launch_bounds__(16 * GDN_ROWS) k_gdn_seq(Shape sh, ScanArgs a, ReqTable rt, int npb) {
  constexpr int VN = Vec16<T>::n;
  typedef typename Vec16<T>::type V;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nh = sh.nh, P = sh.P, N = sh.N;
  const int pb = blockIdx.x % npb, h = (blockIdx.x / npb) % nh, r = blockIdx.x / (npb * nh);
  const int Tr = rt.row0[r + 1] - rt.row0[r];
  if (Tr == 0) return;
  const int grp = h / (nh / sh.G);
  float* xs = reinterpret_cast<float*>(smem);  // [TB][GDN_ROWS]
  float* ks = xs + TB * GDN_ROWS;              // [TB][N]
  float* ag = ks + TB * N;                     // [TB] retention gates
  float* bg = ag + TB;                         // [TB] write gates
  float* iv = bg + TB;                         // [TB] inverse key norms
  const int t = threadIdx.x, nt = blockDim.x;
  const int c16 = t & 15, prow = t >> 4;
  const int p = pb * GDN_ROWS + prow;
  const bool active = p < P;
  float* Hp = reinterpret_cast<float*>(a.state_pool + (int64_t)rt.slot[r] * sh.st_bytes + sh.st_h) +
              ((int64_t)h * P + (active ? p : 0)) * N + c16 * NCH;
  float Hr[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) Hr[j] = active ? Hp[j] : 0.f;
  const float ba = a.dt_bias[h], bb = a.a_log[h];
  const int per = TB / VN;  // 16-byte chunks per feature and block
  const int nblk = (Tr + TB - 1) / TB;
  for (int bl = 0; bl < nblk; ++bl) {
    const int len = min(TB, Tr - bl * TB);
    const int64_t blk = rt.blk0[r] + bl;
    __syncthreads();  // the previous block's LDS is no longer read
    const T* xb = static_cast<const T*>(a.x) + blk * a.xblk;
    for (int c = t; c < GDN_ROWS * per; c += nt) {
      const int fr = c / per, tg = c % per;
      if (pb * GDN_ROWS + fr >= P) continue;
      const V v = *reinterpret_cast<const V*>(xb + tile_off<T>(h * P + pb * GDN_ROWS + fr, tg * VN));
#pragma unroll
      for (int e = 0; e < VN; ++e) xs[(tg * VN + e) * GDN_ROWS + fr] = to_f32(v[e]);
    }
    const T* bb_ = static_cast<const T*>(a.B) + blk * a.bblk;
    for (int c = t; c < N * per; c += nt) {
      const int n = c / per, tg = c % per;
      const V v = *reinterpret_cast<const V*>(bb_ + tile_off<T>(grp * N + n, tg * VN));
#pragma unroll
      for (int e = 0; e < VN; ++e) ks[(tg * VN + e) * N + n] = to_f32(v[e]);
    }
    for (int u = t; u < TB; u += nt) {
      const bool in = u < len;
      const float ra = in ? a.dt[blk * a.dblk + (int64_t)h * TB + u] : 0.f;
      const float rb = in ? a.dt[blk * a.dblk + (int64_t)(nh + h) * TB + u] : 0.f;
      ag[u] = 1.f / (1.f + __expf(-(ra + ba)));
      bg[u] = 1.f / (1.f + __expf(-(rb + bb)));
    }
    __syncthreads();
    // inverse key norms: 16 threads per token (a DPP row), tokens t / 16, t / 16 + nt / 16, ...
    for (int u = t >> 4; u < TB; u += nt >> 4) {
      float ss = 0.f;
      for (int n = c16; n < N; n += 16) ss += ks[u * N + n] * ks[u * N + n];
      ss = row16_sum(ss);
      if (c16 == 0) iv[u] = rsqrtf(ss + 1e-6f);
    }
    __syncthreads();
    // the next token's operands are read while the current one updates the row
    float kn[NCH], inv_n = iv[0], al_n = ag[0], be_n = bg[0], x_n = xs[prow];
#pragma unroll
    for (int j = 0; j < NCH; ++j) kn[j] = ks[c16 * NCH + j];
    for (int u = 0; u < len; ++u) {
      float kv[NCH];
#pragma unroll
      for (int j = 0; j < NCH; ++j) kv[j] = kn[j] * inv_n;
      const float al = al_n, be = be_n, xu = x_n;
      if (u + 1 < TB) {
#pragma unroll
        for (int j = 0; j < NCH; ++j) kn[j] = ks[(u + 1) * N + c16 * NCH + j];
        inv_n = iv[u + 1];
        al_n = ag[u + 1];
        be_n = bg[u + 1];
        x_n = xs[(u + 1) * GDN_ROWS + prow];
      }
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < NCH; ++j) d += Hr[j] * kv[j];
      d = row16_sum(d);
      const float xw = active ? be * xu : 0.f;
      const float bd = be * d;
#pragma unroll
      for (int j = 0; j < NCH; ++j) Hr[j] = al * (Hr[j] - bd * kv[j]) + xw * kv[j];
    }
  }
  if (active)
#pragma unroll
    for (int j = 0; j < NCH; ++j) Hp[j] = Hr[j];
}

size_t gdn_lds_bytes(const Shape& sh) { return sizeof(float) * ((size_t)TB * (GDN_ROWS + sh.N) + 3 * TB); }
bool gdn_supported(const Shape& sh) { return sh.N <= 12 * 16 && gdn_lds_bytes(sh) <= 160 * 1024 - 256; }

template <typename T, int NCH>
static hipError_t launch_gdn_t(const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  const int npb = (sh.P + GDN_ROWS - 1) / GDN_ROWS;
  static std::once_flag once;
  static hipError_t set_err = hipSuccess;
  std::call_once(once, [] {
    set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_gdn_seq<T, NCH>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
  });
  if (set_err != hipSuccess) return set_err;
  hipLaunchKernelGGL((k_gdn_seq<T, NCH>), dim3((unsigned)(rt.n_req * sh.nh * npb)), dim3(16 * GDN_ROWS),
                     gdn_lds_bytes(sh), s, sh, a, rt, npb);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_gdn_dt(const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  switch (sh.N / 16) {
    case 1: return launch_gdn_t<T, 1>(sh, a, rt, s);
    case 2: return launch_gdn_t<T, 2>(sh, a, rt, s);
    case 3: return launch_gdn_t<T, 3>(sh, a, rt, s);
    case 4: return launch_gdn_t<T, 4>(sh, a, rt, s);
    case 5: return launch_gdn_t<T, 5>(sh, a, rt, s);
    case 6: return launch_gdn_t<T, 6>(sh, a, rt, s);
    case 7: return launch_gdn_t<T, 7>(sh, a, rt, s);
    case 8: return launch_gdn_t<T, 8>(sh, a, rt, s);
    case 9: return launch_gdn_t<T, 9>(sh, a, rt, s);
    case 10: return launch_gdn_t<T, 10>(sh, a, rt, s);
    case 11: return launch_gdn_t<T, 11>(sh, a, rt, s);
    default: return launch_gdn_t<T, 12>(sh, a, rt, s);
  }
}

static hipError_t launch_gdn_seq(int dtype, const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  return dtype == HYF_BF16 ? launch_gdn_dt<bf16>(sh, a, rt, s) : launch_gdn_dt<float>(sh, a, rt, s);
}


// ---------------------------------------------------------------------------------------------
// Chunked form of the same rule (chunks of GC = 64 tokens).  Inside a chunk, with H0 the state
// before it, g_t = log alpha_t, G_t = g_1 + ... + g_t and gamma_t = exp(G_t), the rule unrolls to
//   H_t = gamma_t H0 + sum_{s <= t} exp(G_t - G_s) u_s k_s^T,
//   u_t = beta_t (v_t - gamma_t H0 k_t - sum_{s < t} exp(G_t - G_s) (k_s . k_t) u_s).
// With A[t][s] = beta_t exp(G_t - G_s) (k_t . k_s) for s < t (strictly lower triangular) the u_t are
// the rows of U = X - Y H0^T, where (I + A) X = diag(beta) V and (I + A) Y = diag(beta gamma) K
// (rows v_t^T and k_t^T).  The chunk's end state is
//   H_end = gamma_C H0 + (X - Y H0^T)^T Kd,   Kd = rows exp(G_C - G_s) k_s^T.
// X and Y depend on the chunk alone, so every chunk's are solved in parallel (k_gdn_chunk, one
// workgroup per chunk and head: a forward substitution per column of [Y | X]); only the last
// line runs chunk after chunk (k_gdn_chain, one workgroup per request, head and 16 rows of H: a
// row of H evolves on its own given Y, X and Kd).  Tokens past a request's end are no-ops
// (alpha = 1, beta = 0, k = v = 0).
constexpr int GC = 64;

// Record of one (chunk, head) in the workspace, floats: Y [GC][N] (in the chain's MFMA operand
// order, see k_gdn_chunk) | X [GC][P] | kd [GC] | gam_C, padded to 4 floats.  kd_s = exp(G_C - G_s) / sqrt(|B_s|^2 + 1e-6), so Kd[s][n] = kd_s B[s][n].
__host__ __device__ inline int64_t gdn_rec_floats(int N, int P) { return (int64_t)GC * (N + P) + GC + 4; }

// Element (token t < GC of the chunk, feature f of a tiled operand) of a chunk staged tile by
// tile: tile (f / 16, t / KT) of the chunk at LDS tile slot (f / 16) * (GC / KT) + t / KT.
template <typename T>
__device__ __forceinline__ int chunk_tile_idx(int f, int t) {
  constexpr int VN = 16 / (int)sizeof(T), KT = 4 * VN;
  return (((f >> 4) * (GC / KT) + t / KT) * 64 + ((t % KT) / VN) * 16 + (f & 15)) * VN + t % VN;
}

template <typename T>
__global__ void __launch_bounds__(256) k_gdn_chunk(Shape sh, ScanArgs a, ReqTable rt) {
  constexpr int VN = 16 / (int)sizeof(T), KT = 4 * VN;
  typedef typename Vec16<T>::type V;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nh = sh.nh, P = sh.P, N = sh.N;
  const int h = blockIdx.x % nh, q = blockIdx.x / nh;
  int r = 0;
  while (r + 1 < rt.n_req && rt.seg0[r + 1] <= q) ++r;
  const int lc = q - rt.seg0[r];
  const int n_r = rt.row0[r + 1] - rt.row0[r];
  const int t0 = lc * GC;
  const int len = min(GC, n_r - t0);
  const int64_t blk = rt.blk0[r] + t0 / TB;
  const int toff = t0 % TB;
  const int grp = h / (nh / sh.G);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int KP = N + 4, VP = P + 4;
  float* Kt = reinterpret_cast<float*>(smem);  // [GC][KP] k_t (normalized), then scaled rows
  float* Vt = Kt + GC * KP;                    // [GC][VP]
  float* Am = Vt + GC * VP;                    // [GC][GC + 4]
  float* Gs = Am + GC * (GC + 4);              // [GC] G_t
  float* bs = Gs + GC;                         // [GC] beta_t
  float* iv = bs + GC;                         // [GC] inverse key norms
  float* gm = iv + GC;                         // [GC] gamma_t = exp(G_t)
  float* ss = gm + GC;                         // [GC][4] partial squared norms

  // x (= v) and B of the chunk: 16-byte chunks of the tiled layout (VN tokens of one feature),
  // spread token-major; tokens past the request's end are zero
  const T* xb = static_cast<const T*>(a.x) + blk * a.xblk;
  const T* bb = static_cast<const T*>(a.B) + blk * a.bblk;
  // (batches of 8 loads per thread, all in flight before the first is used)
  const int n16 = (N + P) * (GC / VN);
  for (int c0 = 0; c0 < n16; c0 += 8 * 256) {
    V vv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = min(c0 + k * 256 + t, n16 - 1);
      const bool isb = c < N * (GC / VN);
      const int cc = isb ? c : c - N * (GC / VN);
      const int nf = isb ? N : P;
      // feature, first token: consecutive threads take consecutive features (contiguous chunks of a
      // tile, and different LDS banks when spread token-major)
      const int f = cc % nf, tv = (cc / nf) * VN;
      vv[k] = isb ? *reinterpret_cast<const V*>(bb + tile_off<T>((int64_t)grp * N + f, toff + tv))
                  : *reinterpret_cast<const V*>(xb + tile_off<T>((int64_t)h * P + f, toff + tv));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = c0 + k * 256 + t;
      if (c >= n16) continue;
      const bool isb = c < N * (GC / VN);
      const int cc = isb ? c : c - N * (GC / VN);
      const int nf = isb ? N : P;
      const int f = cc % nf, tv = (cc / nf) * VN;
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        const float x = tv + e < len ? to_f32(vv[k][e]) : 0.f;
        if (isb)
          Kt[(tv + e) * KP + f] = x;
        else
          Vt[(tv + e) * VP + f] = x;
      }
    }
  }
  __syncthreads();
  // squared key norms: four threads per token
  {
    const int tk = t >> 2, part = t & 3;
    float acc = 0.f;
    for (int n = part; n < N; n += 4) acc += Kt[tk * KP + n] * Kt[tk * KP + n];
    ss[tk * 4 + part] = acc;
  }
  // gates and the cumulative log-retention (wave 0, one lane per token)
  if (wave == 0) {
    const bool in = lane < len;
    const float za = in ? a.dt[blk * a.dblk + (int64_t)h * TB + toff + lane] + a.dt_bias[h] : 0.f;
    const float zb = in ? a.dt[blk * a.dblk + (int64_t)(nh + h) * TB + toff + lane] + a.a_log[h] : 0.f;
    float g = in ? -softplus_f(-za) : 0.f;  // log sigmoid(za)
    const float be = in ? 1.f / (1.f + __expf(-zb)) : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float u = __shfl_up(g, o, 64);
      if (lane >= o) g += u;
    }
    Gs[lane] = g;
    gm[lane] = __expf(g);
    bs[lane] = be;
  }
  __syncthreads();
  if (t < GC) iv[t] = rsqrtf(ss[t * 4] + ss[t * 4 + 1] + ss[t * 4 + 2] + ss[t * 4 + 3] + 1e-6f);
  __syncthreads();
  for (int idx = t; idx < GC * N; idx += 256) {
    const int tk = idx / N, n = idx % N;
    Kt[tk * KP + n] *= iv[tk];
  }
  __syncthreads();
  // A = strictly lower part of beta_t exp(G_t - G_s) (k_t . k_s): the ten lower 16x16 tiles of the
  // Gram matrix on fp32 MFMAs (lane (i, g) supplies k_{16 ta + i}[4 j + g] and k_{16 tb + i}[4 j + g])
  {
    const int i = lane & 15, g = lane >> 4;
    for (int tile = wave; tile < 10; tile += 4) {
      const int ta = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
      const int tb = tile - ta * (ta + 1) / 2;
      f32x4 ac[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ac[e] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int j4 = 0; j4 < N / 16; ++j4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * j4 + e;
          ac[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(Kt[(16 * ta + i) * KP + 4 * j + g],
                                                      Kt[(16 * tb + i) * KP + 4 * j + g], ac[e], 0, 0, 0);
        }
      const f32x4 acc = (ac[0] + ac[1]) + (ac[2] + ac[3]);
      // lane holds Gram[16 ta + 4 g + rr][16 tb + i]
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int tt = 16 * ta + 4 * g + rr, s = 16 * tb + i;
        Am[tt * (GC + 4) + s] = s < tt ? bs[tt] * __expf(Gs[tt] - Gs[s]) * acc[rr] : 0.f;
        if (ta != tb) Am[s * (GC + 4) + tt] = 0.f;
      }
    }
  }
  __syncthreads();
  // forward substitution, one column of [Y | X] per thread, in place over that column of K (Y) or
  // V (X), which no other thread reads any more:
  //   z_t = rhs_t - sum_{s < t} A[t][s] z_s,  rhs = beta gamma k (Y) or beta v (X).
  // Blocks of 16 rows: the earlier blocks' z come back from LDS 16 at a time, the block's own z stay
  // in registers.
  float* rec = a.part + ((int64_t)q * nh + h) * gdn_rec_floats(N, P);
  for (int col = t; col < N + P; col += 256) {
    const bool isy = col < N;
    float* colp = isy ? Kt + col : Vt + (col - N);
    const int pitch = isy ? KP : VP;
#pragma unroll
    for (int b = 0; b < GC / 16; ++b) {
      float acc[16];
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const int u = 16 * b + tt;
        acc[tt] = bs[u] * (isy ? gm[u] : 1.f) * colp[u * pitch];
      }
#pragma unroll
      for (int sb = 0; sb < b; ++sb) {
        float zp[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) zp[e] = colp[(16 * sb + e) * pitch];
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
          const float* arow = Am + (16 * b + tt) * (GC + 4) + 16 * sb;
#pragma unroll
          for (int s4 = 0; s4 < 16; s4 += 4) {
            const f32x4 am = *reinterpret_cast<const f32x4*>(arow + s4);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[tt] -= am[e] * zp[s4 + e];
          }
        }
      }
#pragma unroll
      for (int tt = 1; tt < 16; ++tt) {
        const float* arow = Am + (16 * b + tt) * (GC + 4) + 16 * b;
#pragma unroll
        for (int s4 = 0; s4 < tt; s4 += 4) {
          const f32x4 am = *reinterpret_cast<const f32x4*>(arow + s4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (s4 + e < tt) acc[tt] -= am[e] * acc[s4 + e];
        }
      }
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) colp[(16 * b + tt) * pitch] = acc[tt];
    }
  }
  __syncthreads();
  // the solved columns to the record in 16-byte stores: Y in the chain's MFMA operand order (element
  // (s, n) at ((s / 16) (N / 16) + n / 16) 256 + (s % 16 + 16 (n % 4)) 4 + (n % 16) / 4, so a chain
  // lane's four k values are one 16-byte load), X row-major
  for (int q4 = t; q4 < GC * N / 4; q4 += 256) {
    const int lf = q4 & 63, bq = q4 >> 6;
    const int sidx = (bq / (N >> 4)) * 16 + (lf & 15);
    const int n0 = (bq % (N >> 4)) * 16 + (lf >> 4);
    f32x4 v;
#pragma unroll
    for (int jr = 0; jr < 4; ++jr) v[jr] = Kt[sidx * KP + n0 + 4 * jr];
    *reinterpret_cast<f32x4*>(rec + 4 * (int64_t)q4) = v;
  }
  for (int q4 = t; q4 < GC * P / 4; q4 += 256) {
    const int sidx = q4 / (P / 4), c4 = q4 % (P / 4);
    *reinterpret_cast<f32x4*>(rec + (int64_t)GC * N + (int64_t)sidx * P + 4 * c4) =
        *reinterpret_cast<const f32x4*>(Vt + sidx * VP + 4 * c4);
  }
  if (t < GC) rec[(int64_t)GC * (N + P) + t] = t < len ? __expf(Gs[GC - 1] - Gs[t]) * iv[t] : 0.f;
  if (t == 0) rec[(int64_t)GC * (N + P) + GC] = __expf(Gs[GC - 1]);
}

// The chain: per (request, head, rows p0 .. p0 + 15 of H), chunk after chunk,
//   S^T = H_rows Y^T (16 x GC),  Z^T = X^T - S^T,  H_rows <- gam_C H_rows + Z^T Kd   (16 x N),
// on fp32 16x16x4 MFMAs, 8 waves (two per SIMD, so one wave's MFMAs cover the other's waits).
// S^T: wave w computes token tile w % 4 over half the k range (w / 4) and leaves a partial in
// LDS; H: wave w computes column tiles w, w + 8, ..., reading Z^T = X^T - S^T_0 - S^T_1 as its A
// operand.  Y goes from the record straight into MFMA operand registers (one 16-byte load per four
// k values, two chunks ahead); X rows, kd and the chunk's key tiles go to a ring of GDN_ST LDS
// stages, GDN_ST - 1 chunks ahead.
constexpr int GDN_ST = 4;
constexpr int GDN_YMAX = 16;  // N / 16 at most (N <= 256)
constexpr int GDN_CW = 8;     // waves of the chain

// Wait until at most n vector-memory operations are outstanding, n rounded down to one of a few
// immediates (waiting for more than needed is always correct).
__device__ __forceinline__ void vm_wait_le(int n) {
  if (n >= 32) vm_wait<32>();
  else if (n >= 24) vm_wait<24>();
  else if (n >= 16) vm_wait<16>();
  else if (n >= 12) vm_wait<12>();
  else if (n >= 8) vm_wait<8>();
  else if (n >= 6) vm_wait<6>();
  else if (n >= 4) vm_wait<4>();
  else if (n >= 3) vm_wait<3>();
  else if (n >= 2) vm_wait<2>();
  else if (n >= 1) vm_wait<1>();
  else vm_wait<0>();
}

template <typename T, int NQ>
__global__ void __launch_bounds__(64 * GDN_CW) k_gdn_chain(Shape sh, ScanArgs a, ReqTable rt, int npb) {
  constexpr int VN = 16 / (int)sizeof(T), KT = 4 * VN;
  constexpr int N = NQ * 16, NQ2 = NQ / 2, NT = 64 * GDN_CW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nh = sh.nh, P = sh.P;
  const int pb = blockIdx.x % npb, h = (blockIdx.x / npb) % nh, r = blockIdx.x / (npb * nh);
  const int n_r = rt.row0[r + 1] - rt.row0[r];
  if (n_r == 0) return;
  const int nc = (n_r + GC - 1) / GC;
  const int p0 = pb * 16;
  const int grp = h / (nh / sh.G);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int ts = wave & 3, kh = wave >> 2;  // S^T token tile and k half of this wave
  const int i = lane & 15, g = lane >> 4;
  constexpr int HP = N + 4, SP = GC + 4;
  const int64_t recf = gdn_rec_floats(N, P);
  // LDS: H rows [16][HP] | S^T partials [2][16][SP] | GDN_ST stages of { X rows [GC][16] | kd [GC] +
  // gam_C (4 spare) | key tiles }
  float* Hs = reinterpret_cast<float*>(smem);
  float* Sp = Hs + 16 * HP;
  constexpr int xbytes = GC * 16 * 4, kbytes = (GC + 4) * 4, bbytes = GC * N * (int)sizeof(T);
  constexpr int stage_bytes = xbytes + kbytes + bbytes;
  char* stage0 = reinterpret_cast<char*>(Sp + 2 * 16 * SP);
  float* Hg = reinterpret_cast<float*>(a.state_pool + (int64_t)rt.slot[r] * sh.st_bytes + sh.st_h) +
              ((int64_t)h * P + p0) * N;
  for (int idx = t; idx < 16 * N; idx += NT) Hs[(idx / N) * HP + idx % N] = Hg[idx];

  auto rec_of = [&](int c) { return a.part + ((int64_t)(rt.seg0[r] + c) * nh + h) * recf; };
  constexpr int NBC = N / 16 * (GC / KT) * 64;  // 16-byte chunks of a chunk's key tiles
  auto issue = [&](int c) {
    char* st = stage0 + (c % GDN_ST) * stage_bytes;
    const float* rec = rec_of(c);
    lds_stage16<NT>(GC * 4, st, [&](int k) { return rec + (int64_t)GC * N + (int64_t)(k >> 2) * P + p0 + 4 * (k & 3); });
    lds_stage16<NT>((GC + 4) / 4, st + xbytes, [&](int k) { return rec + (int64_t)GC * (N + P) + 4 * k; });
    // key tiles of the chunk: tile (fg, jr) is 64 contiguous 16-byte chunks
    const int64_t t0 = (int64_t)c * GC;
    const T* bsrc = static_cast<const T*>(a.B) + (rt.blk0[r] + t0 / TB) * a.bblk;
    const int toff = (int)(t0 % TB);
    lds_stage16<NT>(NBC, st + xbytes + kbytes, [&](int k) {
      const int tile = k >> 6, fg = tile / (GC / KT), jr = tile % (GC / KT);
      return bsrc + tile_off<T>((int64_t)grp * N + 16 * fg, toff + jr * KT) + (k & 63) * VN;
    });
  };
  // copies one stage costs this wave (lds_stage16 issues one per 64-chunk group it owns)
  auto copies = [&](int n) { return n > 64 * wave ? (n - 64 * wave + NT - 1) / NT : 0; };
  const int dw = copies(GC * 4) + copies((GC + 4) / 4) + copies(NBC);
  // Y operands of wave w: rows 16 ts .. + 15, k values 16 jq + 4 jr + g for jq in its half
  auto load_y = [&](int c, f32x4 (&y)[NQ2]) {
    const f32x4* src = reinterpret_cast<const f32x4*>(rec_of(c)) + ((int64_t)ts * NQ + kh * NQ2) * 64 + lane;
#pragma unroll
    for (int jq = 0; jq < NQ2; ++jq) y[jq] = src[jq * 64];
  };
  for (int c = 0; c < GDN_ST - 1 && c < nc; ++c) issue(c);
  f32x4 y0[NQ2], y1[NQ2], y2[NQ2];
  load_y(0, y0);
  if (nc > 1) load_y(1, y1);
  for (int c = 0; c < nc; ++c) {
    // Loads complete in order.  Iteration c needs stage c and Y of chunk c; issued after them are
    // the loads of iteration c - 1 (stage c + 2: dw copies, Y of chunk c + 1: NQ2 loads), or, at
    // c = 0, Y of chunk 1.
    if (c == 0)
      vm_wait_le(nc > 1 ? NQ2 : 0);
    else
      vm_wait_le((c + 2 < nc ? dw : 0) + (c + 1 < nc ? NQ2 : 0));
    // stage c and Y of chunk c are in, H rows of the previous chunk are written; the barrier is the
    // bare instruction (a __syncthreads() fence would wait for the loads still in flight)
    lgkm_wait0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (c + GDN_ST - 1 < nc) issue(c + GDN_ST - 1);
    if (c + 2 < nc) load_y(c + 2, y2);
    const char* st = stage0 + (c % GDN_ST) * stage_bytes;
    const float* Xs = reinterpret_cast<const float*>(st);
    const float* kd = reinterpret_cast<const float*>(st + xbytes);
    const T* Bs = reinterpret_cast<const T*>(st + xbytes + kbytes);
    // partial S^T tile: rows i of H, tokens 16 ts + i, k values of half kh (four chains, one per jr)
    {
      f32x4 ac[4];
#pragma unroll
      for (int jr = 0; jr < 4; ++jr) ac[jr] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jq = 0; jq < NQ2; ++jq)
#pragma unroll
        for (int jr = 0; jr < 4; ++jr)
          ac[jr] = __builtin_amdgcn_mfma_f32_16x16x4f32(Hs[i * HP + 16 * (kh * NQ2 + jq) + 4 * jr + g], y0[jq][jr],
                                                       ac[jr], 0, 0, 0);
      const f32x4 acc = (ac[0] + ac[1]) + (ac[2] + ac[3]);
      // lane holds the partial of S^T[4 g + rr][16 ts + i]
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) Sp[(kh * 16 + 4 * g + rr) * SP + 16 * ts + i] = acc[rr];
    }
    lgkm_wait0();
    __builtin_amdgcn_s_barrier();
    // H columns 16 nt .. + 15: gam_C H + Z^T Kd, A operand Z^T[i][s] = X[s][i] - S^T_0[i][s] -
    // S^T_1[i][s], B operand kd_s B[s][16 nt + i] (s = 4 j + g; the keys past the request's end hold
    // anything, so they are selected away, not multiplied by 0)
    const float gam = kd[GC];
    const int len = min(GC, n_r - c * GC);
    constexpr int TPW = (NQ + GDN_CW - 1) / GDN_CW;
    {
      f32x4 ae[TPW], ao[TPW];
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int nt = min(wave + GDN_CW * k, NQ - 1);  // a wave past the last tile repeats it, unstored
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) ae[k][rr] = gam * Hs[(4 * g + rr) * HP + 16 * nt + i];
        ao[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < GC / 4; ++j) {
        const int s = 4 * j + g;
        const float z = Xs[s * 16 + i] - Sp[i * SP + s] - Sp[(16 + i) * SP + s];
        const float ks = s < len ? kd[s] : 0.f;
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
          const float bv = to_f32(Bs[chunk_tile_idx<T>(16 * min(wave + GDN_CW * k, NQ - 1) + i, s)]);
          const float b = s < len ? ks * bv : 0.f;
          if (j & 1)
            ao[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(z, b, ao[k], 0, 0, 0);
          else
            ae[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(z, b, ae[k], 0, 0, 0);
        }
      }
      // (every wave read all of H before the S^T barrier; after it a wave reads only its own tiles)
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int nt = wave + GDN_CW * k;
        if (nt >= NQ) continue;
        const f32x4 acc = ae[k] + ao[k];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) Hs[(4 * g + rr) * HP + 16 * nt + i] = acc[rr];
      }
    }
#pragma unroll
    for (int jq = 0; jq < NQ2; ++jq) {
      y0[jq] = y1[jq];
      y1[jq] = y2[jq];
    }
  }
  __syncthreads();
  for (int idx = t; idx < 16 * N; idx += NT) Hg[idx] = Hs[(idx / N) * HP + idx % N];
}

static size_t gdn_chunk_lds(const Shape& sh) {
  return sizeof(float) * ((size_t)GC * (sh.N + 4) + (size_t)GC * (sh.P + 4) + (size_t)GC * (GC + 4) + 8 * GC);
}
static size_t gdn_chain_lds(const Shape& sh, int esz) {
  const size_t stage = GC * 16 * 4 + (GC + 4) * 4 + (size_t)GC * sh.N * esz;
  return sizeof(float) * (16 * (size_t)(sh.N + 4) + 2 * 16 * (GC + 4)) + GDN_ST * stage;
}

bool gdn_chunked_supported(const Shape& sh, int esz) {
  return sh.P % 16 == 0 && sh.N % 32 == 0 && sh.N / 16 <= GDN_YMAX && sh.N + sh.P <= 512 &&
         gdn_chunk_lds(sh) <= 160 * 1024 - 256 &&
         gdn_chain_lds(sh, esz) <= 160 * 1024 - 256;
}
int64_t gdn_chunk_record_floats(const Shape& sh) { return gdn_rec_floats(sh.N, sh.P); }

template <typename T>
static hipError_t launch_gdn_chunked_t(const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  static std::once_flag once;
  static hipError_t set_err = hipSuccess;
  std::call_once(once, [] {
    set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_gdn_chunk<T>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
    if (set_err == hipSuccess)
      set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_gdn_chain<T, 2>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
#define HYF_CHAIN_ATTR(NQ)                                                                        \
    if (set_err == hipSuccess)                                                                     \
      set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_gdn_chain<T, NQ>),           \
                                    hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 256);
    HYF_CHAIN_ATTR(4) HYF_CHAIN_ATTR(6) HYF_CHAIN_ATTR(8) HYF_CHAIN_ATTR(10) HYF_CHAIN_ATTR(12)
    HYF_CHAIN_ATTR(14) HYF_CHAIN_ATTR(16)
#undef HYF_CHAIN_ATTR
  });
  if (set_err != hipSuccess) return set_err;
  const int chunks = rt.seg0[rt.n_req];
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gdn_chunk<T>), dim3((unsigned)(chunks * sh.nh)), dim3(256), gdn_chunk_lds(sh), s, sh, a, rt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int npb = sh.P / 16;
  const dim3 grid((unsigned)(rt.n_req * sh.nh * npb));
  const size_t lds = gdn_chain_lds(sh, sizeof(T));
  switch (sh.N / 16) {
    case 2: hipLaunchKernelGGL((k_gdn_chain<T, 2>), grid, dim3(64 * GDN_CW), lds, s, sh, a, rt, npb); break;
    case 4: hipLaunchKernelGGL((k_gdn_chain<T, 4>), grid, dim3(64 * GDN_CW), lds, s, sh, a, rt, npb); break;
    case 6: hipLaunchKernelGGL((k_gdn_chain<T, 6>), grid, dim3(64 * GDN_CW), lds, s, sh, a, rt, npb); break;
    case 8: hipLaunchKernelGGL((k_gdn_chain<T, 8>), grid, dim3(64 * GDN_CW), lds, s, sh, a, rt, npb); break;
    case 10: hipLaunchKernelGGL((k_gdn_chain<T, 10>), grid, dim3(64 * GDN_CW), lds, s, sh, a, rt, npb); break;
    case 12: hipLaunchKernelGGL((k_gdn_chain<T, 12>), grid, dim3(64 * GDN_CW), lds, s, sh, a, rt, npb); break;
    case 14: hipLaunchKernelGGL((k_gdn_chain<T, 14>), grid, dim3(64 * GDN_CW), lds, s, sh, a, rt, npb); break;
    default: hipLaunchKernelGGL((k_gdn_chain<T, 16>), grid, dim3(64 * GDN_CW), lds, s, sh, a, rt, npb); break;
  }
  return hipGetLastError();
}

// rt.seg0 holds each request's first chunk (chunks of GC tokens) when the chunked form runs.
hipError_t launch_gdn_commit(int dtype, const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  if (gdn_chunked_supported(sh, dtype == HYF_BF16 ? 2 : 4))
    return dtype == HYF_BF16 ? launch_gdn_chunked_t<bf16>(sh, a, rt, s) : launch_gdn_chunked_t<float>(sh, a, rt, s);
  return launch_gdn_seq(dtype, sh, a, rt, s);
}

}  // namespace hyf
