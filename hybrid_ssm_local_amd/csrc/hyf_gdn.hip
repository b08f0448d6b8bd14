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

hipError_t launch_gdn_commit(int dtype, const Shape& sh, const ScanArgs& a, const ReqTable& rt, hipStream_t s) {
  return dtype == HYF_BF16 ? launch_gdn_dt<bf16>(sh, a, rt, s) : launch_gdn_dt<float>(sh, a, rt, s);
}

}  // namespace hyf
