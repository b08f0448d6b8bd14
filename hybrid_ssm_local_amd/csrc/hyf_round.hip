// Kernels of one draft/commit round (and the ring/state helpers of a prefill commit).
//
//  k_commit_small  per (request, head, rows of H): folds the round's committed rows into H with
//                  one read-modify-write (chunk form, weights relative to the last row), appends
//                  their (k, v) to the ring, and computes the memory readout of the block rows
//                  from the updated H: mem_j = H . C_q,j + D * v_j.  H is read-only when the call
//                  commits nothing.
//  k_attn          per (request, head, split): softmax attention of the 8 block rows over a
//                  slice of the ring window (or, in the last split, over the block rows
//                  themselves), written as (max, sum, unnormalised output) partials.
//  k_merge         per (request, head): merges the splits, adds mem, stores the output
//                  projection's input, and advances the committed count.
#include <mutex>

#include "hyf_launch.h"

namespace hyf {

constexpr int RB = HYF_BLOCK;   // block rows
constexpr int RMAXC = 16;       // largest per-request commit handled by k_commit_small
constexpr int ATT_KS = 64;      // keys per attention split

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
template <typename T>
__global__ void __launch_bounds__(256) k_commit_small(Shape sh, RoundArgs a, ReqTable rt) {
  __shared__ float Bl[RMAXC][256];
  __shared__ float Cl[RB][256];
  __shared__ float red[RB][256];
  __shared__ float wl[RMAXC];
  __shared__ float decay_s;

  const int nh = sh.nh, P = sh.P, N = sh.N;
  const int r = blockIdx.x / nh, h = blockIdx.x % nh;
  const int slot = rt.slot[r];
  const int grp = h / (nh / sh.G);
  const int tpr = N / 4;                    // threads per H row (float4 each)
  const int rows_wg = 256 / tpr;            // H rows per workgroup
  const int p0 = blockIdx.y * rows_wg;
  const int t = threadIdx.x;
  const int prow = t / tpr, c4 = t % tpr;
  const int p = p0 + prow;
  const bool active = prow < rows_wg && p < P;
  const int nrows = a.do_commit ? rt.row0[r + 1] - rt.row0[r] : 0;
  const int64_t crow0 = rt.row0[r];
  const int64_t brow0 = a.blk_row0 + (int64_t)r * RB;
  const int ld = sh.n_in;

  // stage B rows of the commit and C rows of the block
  for (int idx = t; idx < nrows * N; idx += 256) {
    const int tt = idx / N, n = idx % N;
    Bl[tt][n] = a.proj[(crow0 + tt) * ld + sh.off_b + grp * N + n];
  }
  if (a.do_draft)
    for (int idx = t; idx < RB * N; idx += 256) {
      const int j = idx / N, n = idx % N;
      Cl[j][n] = a.proj[(brow0 + j) * ld + sh.off_c + grp * N + n];
    }
  if (t == 0) {
    // weights relative to the last committed row: w_t = dt_t exp(sum_{tau > t} dt_tau A)
    const float A = -expf(a.a_log[h]);
    float suffix = 0.f;
    for (int tt = nrows - 1; tt >= 0; --tt) {
      const float dt = softplus_f(a.proj[(crow0 + tt) * ld + sh.off_dt + h] + a.dt_bias[h]);
      wl[tt] = dt * expf(suffix);
      suffix += dt * A;
    }
    decay_s = expf(suffix);
  }
  __syncthreads();

  float* Hh = h_ptr(a.state_pool, sh, slot, h);
  f32x4 hv = f32x4{0.f, 0.f, 0.f, 0.f};
  if (active) {
    hv = *reinterpret_cast<const f32x4*>(Hh + (int64_t)p * N + 4 * c4);
    if (nrows > 0) {
      hv *= decay_s;
      for (int tt = 0; tt < nrows; ++tt) {
        const float xv = a.proj[(crow0 + tt) * ld + sh.off_v + h * P + p] * wl[tt];
#pragma unroll
        for (int u = 0; u < 4; ++u) hv[u] += xv * Bl[tt][4 * c4 + u];
      }
      *reinterpret_cast<f32x4*>(Hh + (int64_t)p * N + 4 * c4) = hv;
    }
  }

  if (a.do_draft) {
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      float s = 0.f;
      if (active) {
#pragma unroll
        for (int u = 0; u < 4; ++u) s += hv[u] * Cl[j][4 * c4 + u];
      }
      red[j][t] = s;
    }
    __syncthreads();
    const float D = a.d_skip[h];
    for (int idx = t; idx < RB * rows_wg; idx += 256) {
      const int j = idx / rows_wg, pr = idx % rows_wg;
      const int pp = p0 + pr;
      if (pp >= P) continue;
      float s = 0.f;
      for (int c = 0; c < tpr; ++c) s += red[j][pr * tpr + c];
      const float vj = a.proj[(brow0 + j) * ld + sh.off_v + h * P + pp];
      a.mem[(((int64_t)r * RB + j) * nh + h) * P + pp] = s + D * vj;
    }
  }

  // ring append of this round's rows (first row-tile workgroup of each head)
  if (blockIdx.y == 0 && nrows > 0) {
    const int64_t count = *count_ptr(a.state_pool, sh, slot);
    const int W = sh.W;
    const int first = nrows > W ? nrows - W : 0;
    T* K = ring_ptr<T>(a.state_pool, sh, slot, sh.st_k, h);
    T* V = ring_ptr<T>(a.state_pool, sh, slot, sh.st_v, h);
    for (int idx = t; idx < (nrows - first) * P; idx += 256) {
      const int tt = first + idx / P, pp = idx % P;
      const int64_t s = (count + tt) % W;
      K[s * P + pp] = from_f32<T>(a.proj[(crow0 + tt) * ld + sh.off_k + h * P + pp]);
      V[s * P + pp] = from_f32<T>(a.proj[(crow0 + tt) * ld + sh.off_v + h * P + pp]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) k_attn(Shape sh, RoundArgs a, ReqTable rt) {
  extern __shared__ float dsm[];
  const int nh = sh.nh, P = sh.P;
  const int PK = P + 1;  // key rows padded so consecutive keys fall in different banks
  float* qs = dsm;                    // [8][P]
  float* ks = qs + RB * P;            // [64][P+1]
  float* vs = ks + ATT_KS * PK;       // [64][P]
  float* pl = vs + ATT_KS * P;        // [8][64]

  const int r = blockIdx.x / nh, h = blockIdx.x % nh;
  const int sp = blockIdx.y;
  const int slot = rt.slot[r];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int ld = sh.n_in;
  const int64_t brow0 = a.blk_row0 + (int64_t)r * RB;
  const bool blk = sp == a.n_split - 1;

  int nk;
  if (blk) {
    nk = RB;
  } else {
    const int64_t count = *count_ptr(a.state_pool, sh, slot);
    const int64_t added = a.do_commit ? rt.row0[r + 1] - rt.row0[r] : 0;
    const int64_t tot = count + added;
    const int valid = (int)(tot < sh.W ? tot : sh.W);
    const int k0 = sp * a.keys_per_split;
    nk = valid - k0;
    nk = nk < 0 ? 0 : (nk > a.keys_per_split ? a.keys_per_split : nk);
  }
  float* op = a.att_part + ((((int64_t)r * nh + h) * a.n_split + sp) * RB) * P;
  float* ml = a.att_ml + ((((int64_t)r * nh + h) * a.n_split + sp) * RB) * 2;
  if (nk == 0) {
    for (int idx = t; idx < RB * P; idx += 256) op[idx] = 0.f;
    if (t < RB) {
      ml[2 * t] = -INFINITY;
      ml[2 * t + 1] = 0.f;
    }
    return;
  }

  const float scale = rsqrtf((float)P);
  for (int idx = t; idx < RB * P; idx += 256) {
    const int j = idx / P, pp = idx % P;
    qs[idx] = a.proj[(brow0 + j) * ld + sh.off_q + h * P + pp] * scale;
  }
  if (blk) {
    for (int idx = t; idx < RB * P; idx += 256) {
      const int j = idx / P, pp = idx % P;
      ks[j * PK + pp] = a.proj[(brow0 + j) * ld + sh.off_k + h * P + pp];
      vs[j * P + pp] = a.proj[(brow0 + j) * ld + sh.off_v + h * P + pp];
    }
  } else {
    const T* K = ring_ptr<T>(a.state_pool, sh, slot, sh.st_k, h) + (int64_t)sp * a.keys_per_split * P;
    const T* V = ring_ptr<T>(a.state_pool, sh, slot, sh.st_v, h) + (int64_t)sp * a.keys_per_split * P;
    for (int idx = t; idx < nk * P; idx += 256) {
      const int key = idx / P, pp = idx % P;
      ks[key * PK + pp] = to_f32(K[idx]);
      vs[key * P + pp] = to_f32(V[idx]);
    }
  }
  __syncthreads();

  // scores: lane = key, wave w handles block rows w and w + 4
  const int key = lane;
  float s[2];
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int j = wave + 4 * q2;
    float acc = 0.f;
    if (key < nk) {
      for (int pp = 0; pp < P; ++pp) acc += qs[j * P + pp] * ks[key * PK + pp];
    }
    bool ok = key < nk;
    if (blk && !sh.cross && key != j) ok = false;
    s[q2] = ok ? acc : -INFINITY;
  }
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int j = wave + 4 * q2;
    const float m = wave_max(s[q2]);
    const float e = s[q2] == -INFINITY ? 0.f : expf(s[q2] - m);
    const float l = wave_sum(e);
    pl[j * ATT_KS + key] = e;
    if (lane == 0) {
      ml[2 * j] = m;
      ml[2 * j + 1] = l;
    }
  }
  __syncthreads();
  for (int idx = t; idx < RB * P; idx += 256) {
    const int j = idx / P, pp = idx % P;
    float acc = 0.f;
    for (int k2 = 0; k2 < nk; ++k2) acc += pl[j * ATT_KS + k2] * vs[k2 * P + pp];
    op[idx] = acc;
  }
}

// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) k_merge(Shape sh, RoundArgs a, ReqTable rt) {
  const int nh = sh.nh, P = sh.P;
  const int r = blockIdx.x / nh, h = blockIdx.x % nh;
  const int t = threadIdx.x;
  const float* ml = a.att_ml + (((int64_t)r * nh + h) * a.n_split) * RB * 2;
  const float* op = a.att_part + (((int64_t)r * nh + h) * a.n_split) * RB * P;
  T* out = static_cast<T*>(a.o_in);
  for (int idx = t; idx < RB * P; idx += 256) {
    const int j = idx / P, pp = idx % P;
    float m = -INFINITY;
    for (int s = 0; s < a.n_split; ++s) m = fmaxf(m, ml[(s * RB + j) * 2]);
    float l = 0.f, o = 0.f;
    for (int s = 0; s < a.n_split; ++s) {
      const float ms = ml[(s * RB + j) * 2];
      if (ms == -INFINITY) continue;
      const float f = expf(ms - m);
      l += f * ml[(s * RB + j) * 2 + 1];
      o += f * op[((int64_t)s * RB + j) * P + pp];
    }
    const float att = o / l;
    const float mem = a.mem[(((int64_t)r * RB + j) * nh + h) * P + pp];
    out[((int64_t)r * RB + j) * sh.dq + h * P + pp] = from_f32<T>(att + mem);
  }
  if (h == 0 && t == 0 && a.do_commit) *count_ptr(a.state_pool, sh, rt.slot[r]) += rt.row0[r + 1] - rt.row0[r];
}

// ---------------------------------------------------------------------------------------------
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

// ---------------------------------------------------------------------------------------------
hipError_t launch_commit_small(int dtype, const Shape& sh, const RoundArgs& a, const ReqTable& rt, hipStream_t s) {
  const int rows_wg = 256 / (sh.N / 4);
  dim3 grid((unsigned)rt.n_req * sh.nh, (sh.P + rows_wg - 1) / rows_wg);
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_commit_small<bf16>, grid, dim3(256), 0, s, sh, a, rt);
  else
    hipLaunchKernelGGL(k_commit_small<float>, grid, dim3(256), 0, s, sh, a, rt);
  return hipGetLastError();
}

size_t attn_lds_bytes(const Shape& sh) {
  return sizeof(float) * ((size_t)RB * sh.P + (size_t)ATT_KS * (sh.P + 1) + (size_t)ATT_KS * sh.P + RB * ATT_KS);
}

hipError_t launch_attention(int dtype, const Shape& sh, const RoundArgs& a, const ReqTable& rt, hipStream_t s) {
  dim3 grid((unsigned)rt.n_req * sh.nh, a.n_split);
  const size_t lds = attn_lds_bytes(sh);
  if (lds > 65536) {
    // Above 64 KiB of dynamic LDS the kernel has to opt in (gfx950 has 160 KiB per workgroup).
    // Done once per process with the largest size any shape needs, so later calls (possibly under
    // stream capture) launch only kernels.
    static std::once_flag once;
    static hipError_t set_err = hipSuccess;
    std::call_once(once, [] {
      const int mx = 160 * 1024;
      set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_attn<bf16>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, mx);
      if (set_err == hipSuccess)
        set_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_attn<float>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, mx);
    });
    if (set_err != hipSuccess) return set_err;
  }
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_attn<bf16>, grid, dim3(256), lds, s, sh, a, rt);
  else
    hipLaunchKernelGGL(k_attn<float>, grid, dim3(256), lds, s, sh, a, rt);
  return hipGetLastError();
}

hipError_t launch_merge(int dtype, const Shape& sh, const RoundArgs& a, const ReqTable& rt, hipStream_t s) {
  dim3 grid((unsigned)rt.n_req * sh.nh);
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_merge<bf16>, grid, dim3(256), 0, s, sh, a, rt);
  else
    hipLaunchKernelGGL(k_merge<float>, grid, dim3(256), 0, s, sh, a, rt);
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
