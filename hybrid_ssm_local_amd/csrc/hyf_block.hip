// The full drafter block's own kernels: the pre-norms, the residuals and the SwiGLU gate.  The
// block's matrix products (the layer, w_gate_up, w_down) run through the projection and GEMM
// kernels of the layer.
//
//   h   = x + Layer(RMSNorm(x) * norm1)
//   out = h + (silu(z . w_gate^T) * (z . w_up^T)) . w_down^T,   z = RMSNorm(h) * norm2
//
// Every kernel here is one pass over rows of d_model (or d_ff) elements, HBM-bound and tiny at
// round sizes; a workgroup owns whole rows so the norm's mean square is one in-workgroup sum.
#include "hyf_launch.h"

namespace hyf {

constexpr int BK_THREADS = 256;

// Sum of v over the workgroup (256 threads), returned to every thread.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < BK_THREADS / 64; ++w) s += red[w];
  __syncthreads();  // red may be reused by the caller's next sum
  return s;
}

// y[m] = x[m] / sqrt(mean(x[m]^2) + eps) * g, one workgroup per row.
template <typename TI, typename TO>
__global__ void __launch_bounds__(BK_THREADS) k_rmsnorm(const TI* __restrict__ x, int64_t ldx, const float* __restrict__ g,
                                                      float eps, TO* __restrict__ y, int64_t ldy, int d) {
  __shared__ float red[BK_THREADS / 64];
  const int64_t m = blockIdx.x;
  const TI* xr = x + m * ldx;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += BK_THREADS) {
    const float v = to_f32(xr[i]);
    ss += v * v;
  }
  const float r = rsqrtf(block_sum(ss, red) / (float)d + eps);
  TO* yr = y + m * ldy;
  for (int i = threadIdx.x; i < d; i += BK_THREADS) yr[i] = from_f32<TO>(to_f32(xr[i]) * r * g[i]);
}

// The first residual and the second norm in one pass: h = x + o (fp32, kept for the last residual)
// and z = RMSNorm(h) * g (storage dtype, the MLP's input).
template <typename T>
__global__ void __launch_bounds__(BK_THREADS) k_resid_norm(const T* __restrict__ x, const T* __restrict__ o,
                                                         const float* __restrict__ g, float eps, float* __restrict__ h,
                                                         T* __restrict__ z, int d) {
  __shared__ float red[BK_THREADS / 64];
  const int64_t m = blockIdx.x;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += BK_THREADS) {
    const float v = to_f32(x[m * d + i]) + to_f32(o[m * d + i]);
    h[m * d + i] = v;
    ss += v * v;
  }
  const float r = rsqrtf(block_sum(ss, red) / (float)d + eps);
  // each thread reads back the h values it wrote itself
  for (int i = threadIdx.x; i < d; i += BK_THREADS) z[m * d + i] = from_f32<T>(h[m * d + i] * r * g[i]);
}

// a[m][j] = silu(gu[m][j]) * gu[m][F + j]: the gate columns first, then the up columns.
template <typename T>
__global__ void __launch_bounds__(BK_THREADS) k_swiglu(const float* __restrict__ gu, int F, T* __restrict__ a,
                                                     int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * BK_THREADS + threadIdx.x;
  if (i >= n) return;
  const int64_t m = i / F;
  const int j = (int)(i % F);
  const float gv = gu[m * 2 * F + j], uv = gu[m * 2 * F + F + j];
  a[i] = from_f32<T>(gv / (1.f + __expf(-gv)) * uv);
}

// out = h + y (the second residual), in the storage dtype.
template <typename T>
__global__ void __launch_bounds__(BK_THREADS) k_add_out(const float* __restrict__ h, const float* __restrict__ y,
                                                      T* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * BK_THREADS + threadIdx.x;
  if (i < n) out[i] = from_f32<T>(h[i] + y[i]);
}

hipError_t launch_rmsnorm(int dtype, const void* x, int64_t rows, int d, const float* g, float eps, void* y,
                          hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL((k_rmsnorm<bf16, bf16>), dim3((unsigned)rows), dim3(BK_THREADS), 0, s,
                       static_cast<const bf16*>(x), (int64_t)d, g, eps, static_cast<bf16*>(y), (int64_t)d, d);
  else
    hipLaunchKernelGGL((k_rmsnorm<float, float>), dim3((unsigned)rows), dim3(BK_THREADS), 0, s,
                       static_cast<const float*>(x), (int64_t)d, g, eps, static_cast<float*>(y), (int64_t)d, d);
  return hipGetLastError();
}

hipError_t launch_resid_norm(int dtype, const void* x, const void* o, int64_t rows, int d, const float* g, float eps,
                             float* h, void* z, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_resid_norm<bf16>, dim3((unsigned)rows), dim3(BK_THREADS), 0, s, static_cast<const bf16*>(x),
                       static_cast<const bf16*>(o), g, eps, h, static_cast<bf16*>(z), d);
  else
    hipLaunchKernelGGL(k_resid_norm<float>, dim3((unsigned)rows), dim3(BK_THREADS), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(o), g, eps, h, static_cast<float*>(z),
                       d);
  return hipGetLastError();
}

hipError_t launch_swiglu(int dtype, const float* gu, int64_t rows, int F, void* a, hipStream_t s) {
  const int64_t n = rows * F;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + BK_THREADS - 1) / BK_THREADS));
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_swiglu<bf16>, grid, dim3(BK_THREADS), 0, s, gu, F, static_cast<bf16*>(a), n);
  else
    hipLaunchKernelGGL(k_swiglu<float>, grid, dim3(BK_THREADS), 0, s, gu, F, static_cast<float*>(a), n);
  return hipGetLastError();
}

hipError_t launch_add_out(int dtype, const float* h, const float* y, int64_t n, void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + BK_THREADS - 1) / BK_THREADS));
  if (dtype == HYF_BF16)
    hipLaunchKernelGGL(k_add_out<bf16>, grid, dim3(BK_THREADS), 0, s, h, y, static_cast<bf16*>(out), n);
  else
    hipLaunchKernelGGL(k_add_out<float>, grid, dim3(BK_THREADS), 0, s, h, y, static_cast<float*>(out), n);
  return hipGetLastError();
}

}  // namespace hyf
