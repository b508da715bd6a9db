// rope.hip -- rotary position embedding fused with per-head E4M3 quantisation.
//
// The AWS post "Amazon SageMaker AI 上的 Mixture-of-Experts 内核工程优化",
// section "Triton JIT recompilation elimination", names a serving kernel that
// fuses rotary position embedding with FP8 quantisation per head and
// recompiled for every new token count.  The pages give no formula; the
// reading implemented here:
//   x [T, nH, D] (bf16 or f32), D a multiple of 16; positions pos [T];
//   inverse frequencies inv_freq [D/2] (fp32, an input);
//   angle a(t, i) = fl32(pos[t] * inv_freq[i]), negated for the inverse
//   rotation; pair (u, v) = (x[t,h,i], x[t,h,i+D/2]) (halves) or
//   (x[t,h,2i], x[t,h,2i+1]) (interleaved) becomes
//     u' = u cos a - v sin a,   v' = v cos a + u sin a;
//   one scale per head over the call's tokens, s_h = fl32(amax|y| / 448)
//   (1 when 0) or a static per-head scale; codes E4M3(fl32(y / s_h)).
// The GPU rotates in fp32 (sincosf of the fp32 angle, fused multiply-adds).
//
// Layout of the work: a unit is 16 outputs of one (token, head): 8 pairs of
// consecutive pair indices.  A workgroup takes TB tokens at a time; their
// cos/sin values are computed once into LDS and shared by the nH heads.
//   rope_amax_kernel   rotate, per-head max |y| of its tokens -> partials[wg][h]
//   rope_scale_kernel  one workgroup: s_h from the partials -> scales[h]
//   rope_quant_kernel  rotate again (x from L2 / the MALL), codes of y / s_h
//   rope_one_kernel    both passes in one workgroup (small batches: one launch)
// With static scales only rope_quant_kernel runs.  T is only ever a kernel
// argument.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kRopeThreads = 256;
constexpr int kRopeOneThreads = 1024;
constexpr int kRopeMaxAngles = 1024;  // TB * D/2 per iteration
constexpr int kRopeMaxGrid = 1024;
constexpr int kRopeMaxHeads = 256;
constexpr long long kRopeOneMax = 1LL << 18;  // elements handled by one workgroup

struct RopeArgs {
  const void* x;
  const int32_t* pos;
  const float* inv_freq;
  int T, nH, D, TB, TB1, inverse;  // TB / TB1: tokens per block (grid / one workgroup)
  const float* static_scales;
  uint8_t* codes;
  float* scales;    // [nH] written
  float* partials;  // [grid][nH]
};

// Eight consecutive elements of x starting at element i (16-byte aligned).
template <int XT>
__device__ __forceinline__ void rope_load8(const void* x, size_t i, float v[8]) {
  if (XT == DT_BF16) {
    const i32x4 q = ld16(reinterpret_cast<const uint16_t*>(x) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32((uint32_t)q[j] & 0xffffu);
      v[2 * j + 1] = bf16_bits_to_f32((uint32_t)q[j] >> 16);
    }
  } else {
    const i32x4 p = ld16(reinterpret_cast<const float*>(x) + i);
    const i32x4 q = ld16(reinterpret_cast<const float*>(x) + i + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = __int_as_float(p[j]);
      v[4 + j] = __int_as_float(q[j]);
    }
  }
}

// cos/sin of the angles of tokens [t0, t0 + nt) into cs[tl * D/2 + i].
__device__ __forceinline__ void rope_angles(const RopeArgs& a, int t0, int nt, float2* cs) {
  const int half = a.D >> 1;
  for (int k = threadIdx.x; k < nt * half; k += blockDim.x) {
    const int tl = k / half, i = k - tl * half;
    float ang = (float)a.pos[t0 + tl] * a.inv_freq[i];
    if (a.inverse) ang = -ang;
    float s, c;
    sincosf(ang, &s, &c);
    cs[k] = make_float2(c, s);
  }
}

// The 16 outputs of unit g of head h of token t.  Halves pairing: y[0..7]
// are positions 8g..8g+7, y[8..15] the same positions + D/2.  Interleaved:
// y[0..15] are positions 16g..16g+15.
template <int XT, bool IL>
__device__ __forceinline__ void rope_unit(const RopeArgs& a, int t, int h, int g,
                                          const float2* cs, float y[16]) {
  const size_t row = ((size_t)t * a.nH + h) * a.D;
  float p[8], q[8];
  if (IL) {
    rope_load8<XT>(a.x, row + 16 * g, p);
    rope_load8<XT>(a.x, row + 16 * g + 8, q);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float u = j < 4 ? p[2 * j] : q[2 * j - 8];
      const float v = j < 4 ? p[2 * j + 1] : q[2 * j - 7];
      const float2 c = cs[8 * g + j];
      y[2 * j] = __builtin_fmaf(u, c.x, -(v * c.y));
      y[2 * j + 1] = __builtin_fmaf(v, c.x, u * c.y);
    }
  } else {
    rope_load8<XT>(a.x, row + 8 * g, p);
    rope_load8<XT>(a.x, row + (a.D >> 1) + 8 * g, q);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float2 c = cs[8 * g + j];
      y[j] = __builtin_fmaf(p[j], c.x, -(q[j] * c.y));
      y[8 + j] = __builtin_fmaf(q[j], c.x, p[j] * c.y);
    }
  }
}

template <bool IL>
__device__ __forceinline__ void rope_store(const RopeArgs& a, int t, int h, int g, const float y[16],
                                           float s) {
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; ++j) w[j >> 2] |= f32_to_e4m3(y[j] / s) << (8 * (j & 3));
  uint8_t* row = a.codes + ((size_t)t * a.nH + h) * a.D;
  if (IL) {
    *reinterpret_cast<uint4*>(row + 16 * g) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<uint2*>(row + 8 * g) = make_uint2(w[0], w[1]);
    *reinterpret_cast<uint2*>(row + (a.D >> 1) + 8 * g) = make_uint2(w[2], w[3]);
  }
}

// Pass 1 over this workgroup's token blocks: per-head max |y| into am (LDS,
// as the bits of non-negative floats, whose integer order is their order).
// The block's (token, unit) items are spread over the threads.  cs is two
// buffers of kRopeMaxAngles: a buffer is rewritten two blocks after its use,
// past a barrier every thread has reached.
template <int XT, bool IL>
__device__ __forceinline__ void rope_pass_amax(const RopeArgs& a, int TB, int tb0, int tbstep,
                                               float2* cs, uint32_t* am) {
  const int gph = a.D >> 4, upt = a.nH * gph;
  int it = 0;
  for (int t0 = tb0 * TB; t0 < a.T; t0 += tbstep * TB, ++it) {
    const int nt = min(TB, a.T - t0);
    float2* c = cs + (it & 1) * kRopeMaxAngles;
    rope_angles(a, t0, nt, c);
    __syncthreads();
    for (int k = threadIdx.x; k < nt * upt; k += blockDim.x) {
      const int tl = k / upt, r = k - tl * upt, h = r / gph, g = r - h * gph;
      float y[16];
      rope_unit<XT, IL>(a, t0 + tl, h, g, c + tl * (a.D >> 1), y);
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) m = fmaxf(m, __builtin_fabsf(y[j]));
      atomicMax(&am[h], __float_as_uint(m));
    }
  }
}

template <int XT, bool IL>
__device__ __forceinline__ void rope_pass_quant(const RopeArgs& a, int TB, int tb0, int tbstep,
                                                float2* cs, const float* sc) {
  const int gph = a.D >> 4, upt = a.nH * gph;
  int it = 0;
  for (int t0 = tb0 * TB; t0 < a.T; t0 += tbstep * TB, ++it) {
    const int nt = min(TB, a.T - t0);
    float2* c = cs + (it & 1) * kRopeMaxAngles;
    rope_angles(a, t0, nt, c);
    __syncthreads();
    for (int k = threadIdx.x; k < nt * upt; k += blockDim.x) {
      const int tl = k / upt, r = k - tl * upt, h = r / gph, g = r - h * gph;
      float y[16];
      rope_unit<XT, IL>(a, t0 + tl, h, g, c + tl * (a.D >> 1), y);
      rope_store<IL>(a, t0 + tl, h, g, y, sc[h]);
    }
  }
}

template <int XT, bool IL>
__global__ __launch_bounds__(kRopeThreads) void rope_amax_kernel(RopeArgs a) {
  __shared__ float2 cs[2 * kRopeMaxAngles];
  __shared__ uint32_t am[kRopeMaxHeads];
  for (int h = threadIdx.x; h < a.nH; h += blockDim.x) am[h] = 0u;
  // (the first barrier inside the pass orders these stores before any atomic)
  rope_pass_amax<XT, IL>(a, a.TB, blockIdx.x, gridDim.x, cs, am);
  __syncthreads();
  for (int h = threadIdx.x; h < a.nH; h += blockDim.x)
    a.partials[(size_t)blockIdx.x * a.nH + h] = __uint_as_float(am[h]);
}

// One workgroup: s_h = fl32(max of the partials / 448), 1 when 0.
__global__ __launch_bounds__(kRopeOneThreads) void rope_scale_kernel(RopeArgs a, int nparts) {
  __shared__ uint32_t am[kRopeMaxHeads];
  for (int h = threadIdx.x; h < a.nH; h += blockDim.x) am[h] = 0u;
  __syncthreads();
  const int per = blockDim.x / a.nH;  // >= 4: nH <= 256
  if ((int)threadIdx.x < per * a.nH) {
    const int h = threadIdx.x % a.nH, c = threadIdx.x / a.nH;
    float m = 0.0f;
    for (int p = c; p < nparts; p += per) m = fmaxf(m, a.partials[(size_t)p * a.nH + h]);
    atomicMax(&am[h], __float_as_uint(m));
  }
  __syncthreads();
  for (int h = threadIdx.x; h < a.nH; h += blockDim.x) {
    const float m = __uint_as_float(am[h]);
    a.scales[h] = (m == 0.0f) ? 1.0f : m / 448.0f;
  }
}

// Pass 2; scales from a.static_scales when given (block 0 copies them to
// a.scales), else from a.scales (written by rope_scale_kernel).
template <int XT, bool IL>
__global__ __launch_bounds__(kRopeThreads) void rope_quant_kernel(RopeArgs a) {
  __shared__ float2 cs[2 * kRopeMaxAngles];
  __shared__ float sc[kRopeMaxHeads];
  const float* src = a.static_scales ? a.static_scales : a.scales;
  for (int h = threadIdx.x; h < a.nH; h += blockDim.x) {
    sc[h] = src[h];
    if (a.static_scales && blockIdx.x == 0) a.scales[h] = src[h];
  }
  // (the first barrier inside the pass orders sc before its reads)
  rope_pass_quant<XT, IL>(a, a.TB, blockIdx.x, gridDim.x, cs, sc);
}

// Both passes in one workgroup (x is read the second time from L2).
template <int XT, bool IL>
__global__ __launch_bounds__(kRopeOneThreads) void rope_one_kernel(RopeArgs a) {
  __shared__ float2 cs[2 * kRopeMaxAngles];
  __shared__ uint32_t am[kRopeMaxHeads];
  __shared__ float sc[kRopeMaxHeads];
  for (int h = threadIdx.x; h < a.nH; h += blockDim.x) am[h] = 0u;
  if (!a.static_scales) rope_pass_amax<XT, IL>(a, a.TB1, 0, 1, cs, am);
  __syncthreads();
  for (int h = threadIdx.x; h < a.nH; h += blockDim.x) {
    float s;
    if (a.static_scales) {
      s = a.static_scales[h];
    } else {
      const float m = __uint_as_float(am[h]);
      s = (m == 0.0f) ? 1.0f : m / 448.0f;
    }
    sc[h] = s;
    a.scales[h] = s;
  }
  // every thread is past the last use of both cs buffers (barrier above)
  rope_pass_quant<XT, IL>(a, a.TB1, 0, 1, cs, sc);
}

size_t rope_workspace_bytes(int T, int nH, int D) {
  (void)T;
  (void)D;
  return (size_t)kRopeMaxGrid * nH * sizeof(float);
}

template <int XT, bool IL>
static int rope_launch(RopeArgs a, hipStream_t st) {
  const long long n = (long long)a.T * a.nH * a.D;
  if (n <= kRopeOneMax) {
    hipLaunchKernelGGL((rope_one_kernel<XT, IL>), dim3(1), dim3(kRopeOneThreads), 0, st, a);
    return (int)hipGetLastError();
  }
  const int blocks = (a.T + a.TB - 1) / a.TB;
  const int g = blocks < kRopeMaxGrid ? blocks : kRopeMaxGrid;
  if (!a.static_scales) {
    hipLaunchKernelGGL((rope_amax_kernel<XT, IL>), dim3(g), dim3(kRopeThreads), 0, st, a);
    int err = (int)hipGetLastError();
    if (err) return err;
    hipLaunchKernelGGL(rope_scale_kernel, dim3(1), dim3(kRopeOneThreads), 0, st, a, g);
    err = (int)hipGetLastError();
    if (err) return err;
  }
  hipLaunchKernelGGL((rope_quant_kernel<XT, IL>), dim3(g), dim3(kRopeThreads), 0, st, a);
  return (int)hipGetLastError();
}

int launch_rope_quant(const void* x, int xt, const int32_t* pos, const float* inv_freq, int T,
                      int nH, int D, int interleaved, int inverse, const float* static_scales,
                      uint8_t* codes, float* scales, void* ws, hipStream_t st) {
  RopeArgs a{};
  a.x = x;
  a.pos = pos;
  a.inv_freq = inv_freq;
  a.T = T;
  a.nH = nH;
  a.D = D;
  a.inverse = inverse;
  a.static_scales = static_scales;
  a.codes = codes;
  a.scales = scales;
  a.partials = reinterpret_cast<float*>(ws);
  // tokens per block: about four units per thread, the block's angles in one
  // LDS buffer
  const int upt = nH * (D / 16);
  auto tokens_per_block = [&](int threads) {
    int tb = (4 * threads) / upt;
    if (tb < 1) tb = 1;
    if (tb > kRopeMaxAngles / (D / 2)) tb = kRopeMaxAngles / (D / 2);
    return tb;
  };
  a.TB = tokens_per_block(kRopeThreads);
  a.TB1 = tokens_per_block(kRopeOneThreads);
  if (xt == DT_BF16)
    return interleaved ? rope_launch<DT_BF16, true>(a, st) : rope_launch<DT_BF16, false>(a, st);
  return interleaved ? rope_launch<DT_F32, true>(a, st) : rope_launch<DT_F32, false>(a, st);
}

}  // namespace moe
