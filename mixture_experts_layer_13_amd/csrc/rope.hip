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
// Layout of the work: one wave takes one token at a time.  A unit is 16
// outputs of one head of the token (8 pairs of consecutive pair indices);
// each lane takes units lane, lane + 64, ... of the token, issuing the loads
// of up to rope_items() units before using any of them.  While they are in
// flight the lanes compute the token's D/2 cos/sin values (the position is
// one scalar load, the inverse frequencies sit in registers) into the wave's
// own LDS row, so no workgroup barrier is needed until the end of a kernel.
//   rope_amax_kernel   rotate, per-head max |y| of the workgroup's tokens ->
//                      partials[wg][h]
//   rope_quant_kernel  every workgroup reduces the partials to s_h, rotates
//                      again (x from L2 / the MALL) and writes the codes
//   rope_one_kernel    both passes in one workgroup (small batches: one launch)
// With static scales only rope_quant_kernel runs.  T is only ever a kernel
// argument.
//
// The codes: e4m3_codes4 (common.hpp: the correctly rounded quotient
// without a division per element, the hardware conversion).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kRopeThreads = 1024;
constexpr int kRopeWaves = kRopeThreads / kWave;
constexpr int kRopeMaxHalf = 256;                    // D <= 512
constexpr int kRopeAnglesPerLane = kRopeMaxHalf / kWave;
constexpr int kRopeMaxGrid = 256;                    // workgroups of a pass (partials per head)
constexpr int kRopeMaxHeads = 256;
constexpr long long kRopeOneMax = 1LL << 15;         // elements handled by one workgroup

// Units per lane and sweep: four with bf16 x, two with f32 x (the same 128
// bytes of loads in flight per lane).
template <int XT>
constexpr int rope_items() {
  return XT == DT_BF16 ? 4 : 2;
}

struct RopeArgs {
  const void* x;
  const int32_t* pos;
  const float* inv_freq;
  int T, nH, D, inverse;
  const float* static_scales;
  uint8_t* codes;
  float* scales;    // [nH] written
  float* partials;  // [grid][nH]
};

// Raw bits of unit g of head h of token t: bf16 x takes two 16-byte loads
// (p then q), f32 four.  Halves pairing: p holds positions 8g..8g+7 and q the
// same positions + D/2; interleaved: p and q hold positions 16g..16g+15.
template <int XT, bool IL>
__device__ __forceinline__ void rope_load(const RopeArgs& a, int t, int h, int g, i32x4 raw[4]) {
  const size_t row = ((size_t)t * a.nH + h) * a.D;
  const size_t ip = row + (IL ? 16 * g : 8 * g);
  const size_t iq = IL ? ip + 8 : row + (a.D >> 1) + 8 * g;
  if (XT == DT_BF16) {
    raw[0] = ld16(reinterpret_cast<const uint16_t*>(a.x) + ip);
    raw[1] = ld16(reinterpret_cast<const uint16_t*>(a.x) + iq);
  } else {
    raw[0] = ld16(reinterpret_cast<const float*>(a.x) + ip);
    raw[1] = ld16(reinterpret_cast<const float*>(a.x) + ip + 4);
    raw[2] = ld16(reinterpret_cast<const float*>(a.x) + iq);
    raw[3] = ld16(reinterpret_cast<const float*>(a.x) + iq + 4);
  }
}

template <int XT>
__device__ __forceinline__ void rope_unpack8(const i32x4* raw, float v[8]) {
  if (XT == DT_BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32((uint32_t)raw[0][j] & 0xffffu);
      v[2 * j + 1] = bf16_bits_to_f32((uint32_t)raw[0][j] >> 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = __int_as_float(raw[0][j]);
      v[4 + j] = __int_as_float(raw[1][j]);
    }
  }
}

// The 16 outputs of a unit from its raw bits (cs: the token's cos/sin row).
// Halves pairing: y[0..7] are positions 8g..8g+7, y[8..15] the same + D/2;
// interleaved: y[0..15] are positions 16g..16g+15.
template <int XT, bool IL>
__device__ __forceinline__ void rope_rotate(const i32x4 raw[4], int g, const float2* cs, float y[16]) {
  float p[8], q[8];
  rope_unpack8<XT>(raw, p);
  rope_unpack8<XT>(raw + (XT == DT_BF16 ? 1 : 2), q);
  if (IL) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float u = j < 4 ? p[2 * j] : q[2 * j - 8];
      const float v = j < 4 ? p[2 * j + 1] : q[2 * j - 7];
      const float2 c = cs[8 * g + j];
      y[2 * j] = __builtin_fmaf(u, c.x, -(v * c.y));
      y[2 * j + 1] = __builtin_fmaf(v, c.x, u * c.y);
    }
  } else {
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
                                           float s, float r) {
  const bool fast = e4m3_fast_scale(s, r);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = e4m3_codes4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3], s, r, fast);
  uint8_t* row = a.codes + ((size_t)t * a.nH + h) * a.D;
  if (IL) {
    *reinterpret_cast<uint4*>(row + 16 * g) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<uint2*>(row + 8 * g) = make_uint2(w[0], w[1]);
    *reinterpret_cast<uint2*>(row + (a.D >> 1) + 8 * g) = make_uint2(w[2], w[3]);
  }
}

// Lane state kept for the whole kernel: inv_freq[lane + 64 j].
struct RopeLane {
  float invf[kRopeAnglesPerLane];
};

__device__ __forceinline__ RopeLane rope_lane(const RopeArgs& a) {
  RopeLane L;
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int j = 0; j < kRopeAnglesPerLane; ++j) {
    const int i = lane + kWave * j;
    L.invf[j] = i < (a.D >> 1) ? a.inv_freq[i] : 0.0f;
  }
  return L;
}

// cos/sin of token t's D/2 angles into the wave's LDS row cs.
__device__ __forceinline__ void rope_token_angles(const RopeArgs& a, const RopeLane& L, int t,
                                                  float2* cs) {
  const int lane = threadIdx.x & (kWave - 1);
  const float p = (float)a.pos[t];  // t is uniform over the wave: one scalar load
#pragma unroll
  for (int j = 0; j < kRopeAnglesPerLane; ++j) {
    const int i = lane + kWave * j;
    if (i < (a.D >> 1)) {
      float ang = p * L.invf[j];
      if (a.inverse) ang = -ang;
      float s, c;
      sincosf(ang, &s, &c);
      cs[i] = make_float2(c, s);
    }
  }
}

// Orders a wave's own LDS writes before its later reads (and reads before
// later writes): the wave's lanes run in lockstep, so a wave-scope fence
// around a wave barrier suffices.
__device__ __forceinline__ void rope_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One pass of a wave over its tokens (w0, w0 + wstep, ...).  QUANT = false:
// per-head max |y| into am (LDS, as the bits of non-negative floats, whose
// integer order is their order).  QUANT = true: the codes of y / sc[h]
// (rc[h] = fl32(1 / sc[h])).  cs is the wave's own LDS row.
template <int XT, bool IL, bool QUANT>
__device__ __forceinline__ void rope_wave_pass(const RopeArgs& a, const RopeLane& L, int w0,
                                               int wstep, float2* cs, uint32_t* am,
                                               const float* sc, const float* rc) {
  constexpr int NI = rope_items<XT>();
  const int lane = threadIdx.x & (kWave - 1);
  const int gph = a.D >> 4, upt = a.nH * gph;
  for (int t = w0; t < a.T; t += wstep) {
    for (int base = 0; base < upt; base += NI * kWave) {
      int hs[NI], gs[NI];
      bool live[NI];
      i32x4 raw[NI][4];
#pragma unroll
      for (int s = 0; s < NI; ++s) {  // every load first
        const int r = base + lane + s * kWave;
        live[s] = r < upt;
        const int rr = live[s] ? r : 0;  // a unit past the token reads unit 0
        hs[s] = rr / gph;
        gs[s] = rr - hs[s] * gph;
        rope_load<XT, IL>(a, t, hs[s], gs[s], raw[s]);
      }
      if (base == 0) {
        rope_token_angles(a, L, t, cs);
        rope_wave_sync();
      }
#pragma unroll
      for (int s = 0; s < NI; ++s) {
        float y[16];
        rope_rotate<XT, IL>(raw[s], gs[s], cs, y);
        if (QUANT) {
          if (live[s]) rope_store<IL>(a, t, hs[s], gs[s], y, sc[hs[s]], rc[hs[s]]);
        } else {
          float m = 0.0f;
#pragma unroll
          for (int j = 0; j < 16; ++j) m = fmaxf(m, __builtin_fabsf(y[j]));
          if (live[s]) atomicMax(&am[hs[s]], __float_as_uint(m));
        }
      }
    }
    rope_wave_sync();  // the next token's angles overwrite cs
  }
}

template <int XT, bool IL>
__global__ __launch_bounds__(kRopeThreads) void rope_amax_kernel(RopeArgs a) {
  __shared__ float2 cs[kRopeWaves][kRopeMaxHalf];
  __shared__ uint32_t am[kRopeMaxHeads];
  for (int h = threadIdx.x; h < a.nH; h += blockDim.x) am[h] = 0u;
  const RopeLane L = rope_lane(a);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), waves = blockDim.x / kWave;
  rope_wave_pass<XT, IL, false>(a, L, blockIdx.x * waves + wave, gridDim.x * waves, cs[wave], am,
                                nullptr, nullptr);
  __syncthreads();
  for (int h = threadIdx.x; h < a.nH; h += blockDim.x)
    a.partials[(size_t)blockIdx.x * a.nH + h] = __uint_as_float(am[h]);
}

// s_h and its reciprocal into sc / rc from the nparts partials (static
// scales when given); block 0 writes the scales out.  Ends with a barrier.
__device__ __forceinline__ void rope_scales(const RopeArgs& a, int nparts, uint32_t* am, float* sc,
                                            float* rc) {
  if (!a.static_scales) {
    for (int h = threadIdx.x; h < a.nH; h += blockDim.x) am[h] = 0u;
    __syncthreads();
    const int per = blockDim.x / a.nH;  // >= 4: nH <= 256
    if ((int)threadIdx.x < per * a.nH) {
      const int h = threadIdx.x % a.nH;
      float m = 0.0f;
      for (int p = threadIdx.x / a.nH; p < nparts; p += per)
        m = fmaxf(m, a.partials[(size_t)p * a.nH + h]);
      atomicMax(&am[h], __float_as_uint(m));
    }
    __syncthreads();
  }
  for (int h = threadIdx.x; h < a.nH; h += blockDim.x) {
    float s;
    if (a.static_scales) {
      s = a.static_scales[h];
    } else {
      const float m = __uint_as_float(am[h]);
      s = (m == 0.0f) ? 1.0f : m / 448.0f;
    }
    sc[h] = s;
    rc[h] = 1.0f / s;
    if (blockIdx.x == 0) a.scales[h] = s;
  }
  __syncthreads();
}

template <int XT, bool IL>
__global__ __launch_bounds__(kRopeThreads) void rope_quant_kernel(RopeArgs a, int nparts) {
  __shared__ float2 cs[kRopeWaves][kRopeMaxHalf];
  __shared__ uint32_t am[kRopeMaxHeads];
  __shared__ float sc[kRopeMaxHeads], rc[kRopeMaxHeads];
  const RopeLane L = rope_lane(a);
  rope_scales(a, nparts, am, sc, rc);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), waves = blockDim.x / kWave;
  rope_wave_pass<XT, IL, true>(a, L, blockIdx.x * waves + wave, gridDim.x * waves, cs[wave],
                               nullptr, sc, rc);
}

// Both passes in one workgroup (x is read the second time from L2).
template <int XT, bool IL>
__global__ __launch_bounds__(kRopeThreads) void rope_one_kernel(RopeArgs a) {
  __shared__ float2 cs[kRopeWaves][kRopeMaxHalf];
  __shared__ uint32_t am[kRopeMaxHeads];
  __shared__ float sc[kRopeMaxHeads], rc[kRopeMaxHeads];
  for (int h = threadIdx.x; h < a.nH; h += blockDim.x) am[h] = 0u;
  const RopeLane L = rope_lane(a);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), waves = blockDim.x / kWave;
  if (!a.static_scales)
    rope_wave_pass<XT, IL, false>(a, L, wave, waves, cs[wave], am, nullptr, nullptr);
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
    rc[h] = 1.0f / s;
    a.scales[h] = s;
  }
  __syncthreads();
  rope_wave_pass<XT, IL, true>(a, L, wave, waves, cs[wave], nullptr, sc, rc);
}

size_t rope_workspace_bytes(int T, int nH, int D) {
  (void)T;
  (void)D;
  return (size_t)kRopeMaxGrid * nH * sizeof(float);
}

template <int XT, bool IL>
static int rope_launch(const RopeArgs& a, hipStream_t st) {
  const long long n = (long long)a.T * a.nH * a.D;
  if (n <= kRopeOneMax) {
    hipLaunchKernelGGL((rope_one_kernel<XT, IL>), dim3(1), dim3(kRopeThreads), 0, st, a);
    return (int)hipGetLastError();
  }
  // one token per wave at a time: enough workgroups to give every wave a
  // token, at most one per CU (and kRopeMaxGrid)
  long long g = ((long long)a.T + kRopeWaves - 1) / kRopeWaves;
  const int cus = device_cu_count();
  if (g > cus) g = cus;
  if (g > kRopeMaxGrid) g = kRopeMaxGrid;
  if (!a.static_scales) {
    hipLaunchKernelGGL((rope_amax_kernel<XT, IL>), dim3((unsigned)g), dim3(kRopeThreads), 0, st, a);
    const int err = (int)hipGetLastError();
    if (err) return err;
  }
  hipLaunchKernelGGL((rope_quant_kernel<XT, IL>), dim3((unsigned)g), dim3(kRopeThreads), 0, st, a,
                     (int)g);
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
  if (xt == DT_BF16)
    return interleaved ? rope_launch<DT_BF16, true>(a, st) : rope_launch<DT_BF16, false>(a, st);
  return interleaved ? rope_launch<DT_F32, true>(a, st) : rope_launch<DT_F32, false>(a, st);
}

}  // namespace moe
