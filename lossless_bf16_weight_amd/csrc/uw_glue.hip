// libuw MLP glue kernels for MI355X (gfx950): SwiGLU between the up/gate and down projections
// and the weightless RMS norm feeding the next layer of a decode step.
#include "uw_device.h"

namespace uw {

// =========================================================================================
// MLP glue (SwiGLU between up/gate and down; RMS norm feeding the next layer)
// =========================================================================================

__global__ void k_swiglu(const float* g, const float* u, uint16_t* h, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    h[i] = swiglu1(g[i], u[i]);
}

// Four elements a thread (count % 4 == 0, 16-byte aligned g and u, 8-byte aligned h).
__global__ void k_swiglu4(const floatx4* g, const floatx4* u, u32x2* h, int64_t count4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count4; i += (int64_t)gridDim.x * blockDim.x) {
    const floatx4 gv = g[i], uv = u[i];
    h[i] = u32x2{(uint32_t)swiglu1(gv[0], uv[0]) | ((uint32_t)swiglu1(gv[1], uv[1]) << 16),
                 (uint32_t)swiglu1(gv[2], uv[2]) | ((uint32_t)swiglu1(gv[3], uv[3]) << 16)};
  }
}

// One 1024-thread workgroup a row, V float4 vectors a thread held in registers between the
// sum of squares and the scaling (n % 4 == 0, n <= 4096 * V).  Fixed reduction order: each
// thread's vectors in order, a butterfly inside each wave, then the 16 wave sums in order.
template <int V>
__global__ __launch_bounds__(1024) void k_rmsnorm_v(const float* y, uint16_t* x, int n, float eps) {
  __shared__ float part[16];   // wave sums
  const floatx4* yr = reinterpret_cast<const floatx4*>(y + (size_t)blockIdx.x * n);
  u32x2* xr = reinterpret_cast<u32x2*>(x + (size_t)blockIdx.x * n);
  const int n4 = n >> 2;
  floatx4 v[V];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = (int)threadIdx.x + j * 1024;
    v[j] = i < n4 ? yr[i] : floatx4{0.f, 0.f, 0.f, 0.f};
    ss = rms_acc(ss, v[j]);
  }
  const float scale = rms_scale(part, ss, n, eps);
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = (int)threadIdx.x + j * 1024;
    if (i < n4) xr[i] = rms_pack(v[j], scale);
  }
}

__global__ __launch_bounds__(256) void k_rmsnorm(const float* y, uint16_t* x, int n, float eps) {
  __shared__ float part[4];
  const float* yr = y + (size_t)blockIdx.x * n;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) ss += yr[i] * yr[i];
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float scale = 1.0f / sqrtf(tot / (float)n + eps);
  for (int i = threadIdx.x; i < n; i += 256) x[(size_t)blockIdx.x * n + i] = f32_to_bf16(yr[i] * scale);
}

// Row-wise RMS norm of an fp32 [m, n] y into BF16 x (the vector kernel when the row fits it).
bool rms_vec(const float* y, const uint16_t* x, int n) {
  return n % 4 == 0 && n <= 4 * 4096 && reinterpret_cast<uintptr_t>(y) % 16 == 0 && reinterpret_cast<uintptr_t>(x) % 8 == 0;
}
hipError_t launch_rmsnorm(const float* y, uint16_t* x, int32_t m, int32_t n, float eps, hipStream_t s) {
  const bool vec = rms_vec(y, x, n);
  if (vec && n <= 4096)
    hipLaunchKernelGGL((k_rmsnorm_v<1>), dim3((unsigned)m), dim3(1024), 0, s, y, x, n, eps);
  else if (vec && n <= 8192)
    hipLaunchKernelGGL((k_rmsnorm_v<2>), dim3((unsigned)m), dim3(1024), 0, s, y, x, n, eps);
  else if (vec)
    hipLaunchKernelGGL((k_rmsnorm_v<4>), dim3((unsigned)m), dim3(1024), 0, s, y, x, n, eps);
  else
    hipLaunchKernelGGL(k_rmsnorm, dim3((unsigned)m), dim3(256), 0, s, y, x, n, eps);
  return hipGetLastError();
}

}  // namespace uw

using namespace uw;

extern "C" {

uw_status uw_swiglu(const float* g, const float* u, uint16_t* h, int64_t count, hipStream_t s) {
  if (!g || !u || !h || count < 0) return fail(UW_E_ARG, "bad argument");
  if (count == 0) return UW_OK;
  const bool vec = count % 4 == 0 && reinterpret_cast<uintptr_t>(g) % 16 == 0 && reinterpret_cast<uintptr_t>(u) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(h) % 8 == 0;
  const int64_t items = vec ? count / 4 : count;
  const int64_t blocks = std::min<int64_t>((items + 255) / 256, 4096);
  if (vec)
    hipLaunchKernelGGL(k_swiglu4, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const floatx4*>(g),
                       reinterpret_cast<const floatx4*>(u), reinterpret_cast<u32x2*>(h), items);
  else
    hipLaunchKernelGGL(k_swiglu, dim3((unsigned)blocks), dim3(256), 0, s, g, u, h, count);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(UW_E_HIP, "swiglu launch: %s", hipGetErrorString(e));
  clear_error();
  return UW_OK;
}

uw_status uw_rmsnorm(const float* y, uint16_t* x, int32_t m, int32_t n, float eps, hipStream_t s) {
  if (!y || !x || m < 1 || n < 1) return fail(UW_E_ARG, "bad argument");
  const hipError_t e = launch_rmsnorm(y, x, m, n, eps, s);
  if (e != hipSuccess) return fail(UW_E_HIP, "rmsnorm launch: %s", hipGetErrorString(e));
  clear_error();
  return UW_OK;
}

}  // extern "C"
