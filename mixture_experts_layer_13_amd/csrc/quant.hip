// quant.hip -- FP8 per-tensor activation scaling for E4M3 expert weights.
//
// "Amazon SageMaker AI 上的 Mixture-of-Experts 内核工程优化", section "Backend
// routing for FP8 tensor quantization", covers FP8 per-tensor ("tensor-
// quantized") MoE models; E4M3 (4 exponent, 3 mantissa bits) is named in
// "Amazon SageMaker AI 上的 MoE 内核工程优化实践", section "Triton 后端路由".
// The pages give no formula; the layer uses s = fl32(amax / 448) (1 when
// amax = 0) and codes E4M3(fl32(v / s)), round to nearest even, saturating.
//
//   amax_partial_kernel: per-workgroup max |x| -> partials[g]; workgroup 0
//     also clears the running max of |h| that the gate/up GEMM raises.
//   quant_x_kernel: reduces the partials (or applies a static scale), writes
//     s_x and the E4M3 codes of x.
//   quant_x_one_kernel: the same for up to 1 MiB of x in one workgroup.
//   quant_h_kernel: s_h from the running max (or a static scale), codes of
//     the fp32 intermediate E4M3(fl32(h / s_h)) of the real rows.
// The codes: e4m3_codes4 (common.hpp: the correctly rounded quotient
// without a division per element, the hardware conversion).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kQThreads = 256;

template <int XT>
__device__ __forceinline__ void load8(const void* x, size_t i, float v[8]) {
  if (XT == DT_BF16) {
    i32x4 q = ld16(reinterpret_cast<const uint16_t*>(x) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32((uint32_t)q[j] & 0xffffu);
      v[2 * j + 1] = bf16_bits_to_f32((uint32_t)q[j] >> 16);
    }
  } else {
    i32x4 a = ld16(reinterpret_cast<const float*>(x) + i);
    i32x4 b = ld16(reinterpret_cast<const float*>(x) + i + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = __int_as_float(a[j]);
      v[4 + j] = __int_as_float(b[j]);
    }
  }
}

// Eight codes E4M3(fl32(v / s)), packed little-endian (r = fl32(1 / s),
// fast = e4m3_fast_scale(s, r)).
__device__ __forceinline__ uint2 e4m3_codes8(const float v[8], float s, float r, bool fast) {
  return make_uint2(e4m3_codes4(v[0], v[1], v[2], v[3], s, r, fast), e4m3_codes4(v[4], v[5], v[6], v[7], s, r, fast));
}

template <int NT = kQThreads>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

template <int XT>
__global__ __launch_bounds__(kQThreads) void amax_partial_kernel(
    const void* __restrict__ x, size_t n, float* __restrict__ partials,
    uint32_t* __restrict__ hmax_bits) {
  __shared__ float red[kQThreads / kWave];
  float m = 0.0f;
  for (size_t i = ((size_t)blockIdx.x * kQThreads + threadIdx.x) * 8; i < n;
       i += (size_t)gridDim.x * kQThreads * 8) {
    float v[8];
    load8<XT>(x, i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(v[j]));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) {
    partials[blockIdx.x] = m;
    if (blockIdx.x == 0) *hmax_bits = 0u;
  }
}

// nparts == 0: this is a single-workgroup launch that reduces x itself.
template <int XT>
__global__ __launch_bounds__(kQThreads) void quant_x_kernel(
    const void* __restrict__ x, size_t n, const float* __restrict__ partials,
    int nparts, const float* __restrict__ static_scale, uint8_t* __restrict__ xq,
    float* __restrict__ sx_out, uint32_t* __restrict__ hmax_bits) {
  __shared__ float red[kQThreads / kWave];
  float s;
  if (static_scale) {
    s = *static_scale;
  } else {
    float m = 0.0f;
    if (nparts == 0) {
      for (size_t i = (size_t)threadIdx.x * 8; i < n; i += kQThreads * 8) {
        float v[8];
        load8<XT>(x, i, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(v[j]));
      }
    } else {
      for (int i = threadIdx.x; i < nparts; i += kQThreads) m = fmaxf(m, partials[i]);
    }
    m = block_max(m, red);
    s = (m == 0.0f) ? 1.0f : m / 448.0f;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *sx_out = s;
    if (nparts == 0) *hmax_bits = 0u;
  }
  const float r = 1.0f / s;
  const bool fast = e4m3_fast_scale(s, r);
  for (size_t i = ((size_t)blockIdx.x * kQThreads + threadIdx.x) * 8; i < n;
       i += (size_t)gridDim.x * kQThreads * 8) {
    float v[8];
    load8<XT>(x, i, v);
    *reinterpret_cast<uint2*>(xq + i) = e4m3_codes8(v, s, r, fast);
  }
}

// One 1024-thread workgroup: max |x|, s_x, then the codes (x is read twice,
// the second time from L2).  Up to 32 Ki values one launch beats the
// two-kernel path (measured on E4M3 decode steps: 8 tokens x 4096 126 -> 116
// us against a 256-thread workgroup); from 48 Ki values on the two-kernel
// path wins (12 and 16 tokens: 4-9 us), one CU streaming too slowly.
constexpr int kQOneThreads = 1024;
constexpr size_t kQOneMax = (size_t)1 << 15;  // elements

template <int XT>
__global__ __launch_bounds__(kQOneThreads) void quant_x_one_kernel(
    const void* __restrict__ x, size_t n, uint8_t* __restrict__ xq, float* __restrict__ sx_out,
    uint32_t* __restrict__ hmax_bits) {
  __shared__ float red[kQOneThreads / kWave];
  constexpr size_t kStep = (size_t)kQOneThreads * 8;
  float m = 0.0f;
  size_t i = (size_t)threadIdx.x * 8;
  for (; i + 3 * kStep < n; i += 4 * kStep) {  // four loads in flight per thread
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<XT>(x, i + u * kStep, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(v[u][j]));
  }
  for (; i < n; i += kStep) {
    float v[8];
    load8<XT>(x, i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(v[j]));
  }
  m = block_max<kQOneThreads>(m, red);
  const float s = (m == 0.0f) ? 1.0f : m / 448.0f;
  if (threadIdx.x == 0) {
    *sx_out = s;
    *hmax_bits = 0u;
  }
  const float r = 1.0f / s;
  const bool fast = e4m3_fast_scale(s, r);
  for (size_t k = (size_t)threadIdx.x * 8; k < n; k += kStep) {
    float v[8];
    load8<XT>(x, k, v);
    *reinterpret_cast<uint2*>(xq + k) = e4m3_codes8(v, s, r, fast);
  }
}

// h32: [rows, N] fp32; codes for the rows < *num_rows that hold a pair
// (sorted_ids[row] < P): padding rows are neither read nor written (no
// kernel uses their codes for an output).
__global__ __launch_bounds__(kQThreads) void quant_h_kernel(
    const float* __restrict__ h32, int N, const int32_t* __restrict__ num_rows,
    const int32_t* __restrict__ sorted_ids, int P, const uint32_t* __restrict__ hmax_bits,
    const float* __restrict__ static_scale, uint8_t* __restrict__ hq, float* __restrict__ sh_out) {
  float s;
  if (static_scale) {
    s = *static_scale;
  } else {
    float m = __uint_as_float(*hmax_bits);
    s = (m == 0.0f) ? 1.0f : m / 448.0f;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *sh_out = s;
  const float r = 1.0f / s;
  const bool fast = e4m3_fast_scale(s, r);
  const size_t n = (size_t)(*num_rows) * N;
  for (size_t i = ((size_t)blockIdx.x * kQThreads + threadIdx.x) * 8; i < n;
       i += (size_t)gridDim.x * kQThreads * 8) {
    const int f = sorted_ids[i / N];
    if (f < 0 || f >= P) continue;
    const i32x4 a = ld16(h32 + i), b = ld16(h32 + i + 4);
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = __int_as_float(a[j]);
      v[4 + j] = __int_as_float(b[j]);
    }
    *reinterpret_cast<uint2*>(hq + i) = e4m3_codes8(v, s, r, fast);
  }
}

// Activations quantised beforehand (their codes and scale s_x come in):
// s_x into the forward's scalar and the running max of |h| cleared.
__global__ __launch_bounds__(64) void fwd_prequant_kernel(const float* __restrict__ a1_scale,
                                                          float* __restrict__ sx,
                                                          uint32_t* __restrict__ hmax_bits) {
  if (threadIdx.x == 0) {
    *sx = *a1_scale;
    *hmax_bits = 0u;
  }
}

int launch_fwd_prequant(const float* a1_scale, float* sx, uint32_t* hmax_bits, hipStream_t stream) {
  hipLaunchKernelGGL(fwd_prequant_kernel, dim3(1), dim3(64), 0, stream, a1_scale, sx, hmax_bits);
  return (int)hipGetLastError();
}

int launch_quant_x(const void* x, int xt, size_t n, const float* static_scale,
                   float* partials, uint8_t* xq, float* sx, uint32_t* hmax_bits,
                   hipStream_t stream) {
  // n is a multiple of 128 (K % 128 == 0).
  const size_t per_wg = (size_t)kQThreads * 8;
  size_t want = (n + per_wg - 1) / per_wg;
  if (!static_scale && n <= kQOneMax) {
    if (xt == DT_BF16)
      hipLaunchKernelGGL(quant_x_one_kernel<DT_BF16>, dim3(1), dim3(kQOneThreads), 0, stream, x, n,
                         xq, sx, hmax_bits);
    else
      hipLaunchKernelGGL(quant_x_one_kernel<DT_F32>, dim3(1), dim3(kQOneThreads), 0, stream, x, n,
                         xq, sx, hmax_bits);
    return (int)hipGetLastError();
  }
  if (static_scale) {
    // no reduction: every workgroup quantises its part
    int g = (int)(want < 1024 ? (want ? want : 1) : 1024);
    if (xt == DT_BF16)
      hipLaunchKernelGGL(quant_x_kernel<DT_BF16>, dim3(g), dim3(kQThreads), 0, stream,
                         x, n, partials, 0, static_scale, xq, sx, hmax_bits);
    else
      hipLaunchKernelGGL(quant_x_kernel<DT_F32>, dim3(g), dim3(kQThreads), 0, stream,
                         x, n, partials, 0, static_scale, xq, sx, hmax_bits);
    return (int)hipGetLastError();
  }
  int g = (int)(want < kMaxPartials ? want : kMaxPartials);
  if (xt == DT_BF16) {
    hipLaunchKernelGGL(amax_partial_kernel<DT_BF16>, dim3(g), dim3(kQThreads), 0, stream,
                       x, n, partials, hmax_bits);
    hipLaunchKernelGGL(quant_x_kernel<DT_BF16>, dim3(g), dim3(kQThreads), 0, stream,
                       x, n, partials, g, nullptr, xq, sx, hmax_bits);
  } else {
    hipLaunchKernelGGL(amax_partial_kernel<DT_F32>, dim3(g), dim3(kQThreads), 0, stream,
                       x, n, partials, hmax_bits);
    hipLaunchKernelGGL(quant_x_kernel<DT_F32>, dim3(g), dim3(kQThreads), 0, stream,
                       x, n, partials, g, nullptr, xq, sx, hmax_bits);
  }
  return (int)hipGetLastError();
}

int launch_quant_h(const float* h32, int N, int max_rows, const int32_t* num_rows,
                   const int32_t* sorted_ids, int P, const uint32_t* hmax_bits,
                   const float* static_scale, uint8_t* hq, float* sh, hipStream_t stream) {
  size_t n = (size_t)max_rows * N;
  const size_t per_wg = (size_t)kQThreads * 8;
  size_t want = (n + per_wg - 1) / per_wg;
  int g = (int)(want < 2048 ? (want ? want : 1) : 2048);
  hipLaunchKernelGGL(quant_h_kernel, dim3(g), dim3(kQThreads), 0, stream, h32, N,
                     num_rows, sorted_ids, P, hmax_bits, static_scale, hq, sh);
  return (int)hipGetLastError();
}

}  // namespace moe
