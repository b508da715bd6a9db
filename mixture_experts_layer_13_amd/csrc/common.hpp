// common.hpp -- device helpers shared by the gfx950 kernels of the fused MoE
// layer: number formats, 16-byte memory access, wave reductions and the two
// MFMA operand families (bf16 16x16x32 and E4M3 16x16x128).
//
// MFMA lane layout used throughout (CDNA3/CDNA4 16x16 family, wave64):
//   operand A (16 rows x Kb):  lane l holds row (l % 16), K-group (l / 16);
//   operand B (Kb x 16 cols):  lane l holds col (l % 16), K-group (l / 16);
//   result C (16 x 16, fp32):  lane l holds C[4*(l/16) + i][l % 16], i = 0..3.
// A K-group is 8 bf16 or 32 E4M3 values.  Which K indices a group holds is
// the kernels' choice, as long as A and B use the same assignment (the sum
// over K does not depend on its order): every kernel gives lane group g a
// contiguous run of K so that each lane reads 32 contiguous bytes of a row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };

constexpr int kWave = 64;

// ------------------------------------------------------------ number formats

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// binary32 -> bfloat16, round to nearest even (NaN kept quiet); written
// without a branch so that it stays a few selects in unrolled epilogues.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return (u & 0x7fffffffu) > 0x7f800000u ? ((u >> 16) | 0x40u) : rounded;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two binary32 values -> packed bfloat16 pair (a in the low half), round to
// nearest even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// Whether e4m3_codes4 may use the reciprocal of the scale s.
__device__ __forceinline__ bool e4m3_fast_scale(float s, float r) {
  return s >= 1.17549435e-38f && r <= 3.40282347e+38f;
}

// E4M3(fl32(y / s)) without a division per element: r = fl32(1 / s)
// correctly rounded, fast = e4m3_fast_scale(s, r) (s a positive normal float
// with a finite reciprocal; otherwise every quotient is an IEEE division).
// Markstein's correction step (P. Markstein, IBM J. Res. Dev. 34(1), 1990):
// q = fl32(y r), the residual e = y - s q from one fused multiply-add (exact),
// and fl32(q + e r) is the correctly rounded quotient, except possibly within
// two ulps of a power of two, where the residual can need one bit more than
// binary32 holds.  From 2^-9 (the smallest E4M3 subnormal) up, powers of two
// are E4M3 values, not rounding midpoints, so there the code is that of the
// correctly rounded quotient.  Below 2^-9 lies 2^-10, the midpoint between 0
// and 2^-9: a group of four with a quotient under 2^-9 (zeros among them,
// which so keep their sign) takes the IEEE division for all four, one branch
// per group, and so does a group with an infinite y (its corrected quotient
// is NaN).  Quotients of 448 and more saturate, whatever their last bits.
// The codes come from the hardware
// conversion of the quotient clamped to +-448 (OCP E4M3FN, round to nearest
// even: equal to the IEEE reading at every E4M3 rounding midpoint and its
// fp32 neighbours, both signs, for exact and inexact quotients); a NaN y
// gives a saturated code, not the NaN code.  Four codes, little-endian.
__device__ __forceinline__ uint32_t e4m3_codes4(float y0, float y1, float y2, float y3, float s, float r,
                                                bool fast) {
  float y[4] = {y0, y1, y2, y3}, q[4];
  bool slow = !fast;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float q0 = y[j] * r;
    const float e = __builtin_fmaf(-q0, s, y[j]);
    q[j] = __builtin_fmaf(e, r, q0);
    slow |= !(__builtin_fabsf(q[j]) >= 0x1p-9f);
  }
  if (__builtin_expect(slow, 0)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = y[j] / s;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = __builtin_fminf(__builtin_fmaxf(q[j], -448.0f), 448.0f);
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], v, true);
  return (uint32_t)v;
}


// ----------------------------------------------------------------- memory

__device__ __forceinline__ i32x4 ld16(const void* p) {
  return *reinterpret_cast<const i32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, i32x4 v) {
  *reinterpret_cast<i32x4*>(p) = v;
}

// ------------------------------------------------------------ wave helpers

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// Index of the s-th (0-based) expert with a non-empty segment, scanning
// expert_offsets [E+1]; -1 if fewer than s+1 experts are active.  Every lane
// of the calling wave gets the same answer.
__device__ __forceinline__ int nth_active_expert(const int32_t* __restrict__ off,
                                                 int E, int s) {
  const int lane = threadIdx.x & 63;
  int seen = 0;
  for (int base = 0; base < E; base += kWave) {
    int e = base + lane;
    bool act = (e < E) && (off[e + 1] > off[e]);
    uint64_t bal = __ballot(act);
    int cnt = __popcll(bal);
    if (s < seen + cnt) {
      int want = s - seen;  // the want-th set bit of bal
      int rank = __popcll(bal & lanemask_lt(lane));
      uint64_t hit = __ballot(act && rank == want);
      return base + __ffsll((long long)hit) - 1;
    }
    seen += cnt;
  }
  return -1;
}

// Count the real (non-sentinel) entries of an expert segment; sentinels sit
// only at the tail, so this is also the index of the first padding slot.
__device__ __forceinline__ int segment_count(const int32_t* __restrict__ sorted_ids,
                                             int seg0, int seg1, int P) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  for (int s = seg0; s < seg1; s += kWave) {
    bool real = (s + lane < seg1) && (sorted_ids[s + lane] < P);
    cnt += __popcll(__ballot(real));
  }
  return cnt;
}

// --------------------------------------------------- MFMA operand families
//
// One "step" is the part of K that one MFMA issue group consumes while each
// lane reads 32 contiguous bytes of its row:
//   bf16 family: 16 values per lane -> two 16x16x32 MFMAs, step = 64 of K;
//   E4M3 family: 32 codes per lane  -> one 16x16x128 MFMA,  step = 128 of K.

struct OpBF {
  bf16x8 v[2];
};
struct OpF8 {
  i32x8 v;
};

template <int SRC>
struct Family;  // SRC = storage dtype of the operand in memory
template <>
struct Family<DT_BF16> {
  using Op = OpBF;
  static constexpr int kPerLane = 16;  // K values per lane per step
  static constexpr int kBytes = 2;     // storage bytes per value
};
template <>
struct Family<DT_F32> {
  using Op = OpBF;
  static constexpr int kPerLane = 16;
  static constexpr int kBytes = 4;
};
template <>
struct Family<DT_E4M3> {
  using Op = OpF8;
  static constexpr int kPerLane = 32;
  static constexpr int kBytes = 1;
};

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// 8 fp32 -> 8 bf16 (round to nearest even) packed in an i32x4.
__device__ __forceinline__ i32x4 pack_bf16x8(i32x4 a, i32x4 b) {
  i32x4 r;
  r[0] = (int)(f32_to_bf16_bits(__int_as_float(a[0])) | (f32_to_bf16_bits(__int_as_float(a[1])) << 16));
  r[1] = (int)(f32_to_bf16_bits(__int_as_float(a[2])) | (f32_to_bf16_bits(__int_as_float(a[3])) << 16));
  r[2] = (int)(f32_to_bf16_bits(__int_as_float(b[0])) | (f32_to_bf16_bits(__int_as_float(b[1])) << 16));
  r[3] = (int)(f32_to_bf16_bits(__int_as_float(b[2])) | (f32_to_bf16_bits(__int_as_float(b[3])) << 16));
  return r;
}

// Raw 32 bytes (two or four 16-byte loads) of one lane's step.
template <int SRC>
struct Raw {
  i32x4 q[Family<SRC>::kPerLane * Family<SRC>::kBytes / 16];
};

template <int SRC>
__device__ __forceinline__ Raw<SRC> load_raw(const void* p) {
  Raw<SRC> r;
  const char* c = reinterpret_cast<const char*>(p);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(r.q) / 16); ++i) r.q[i] = ld16(c + 16 * i);
  return r;
}

// Streaming variant for data read exactly once (expert weights): non-temporal
// loads keep it from displacing reusable lines (activations, h) in L2.
template <int SRC>
__device__ __forceinline__ Raw<SRC> load_raw_nt(const void* p) {
  Raw<SRC> r;
  const i32x4* c = reinterpret_cast<const i32x4*>(p);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(r.q) / 16); ++i) r.q[i] = __builtin_nontemporal_load(c + i);
  return r;
}

template <int SRC>
__device__ __forceinline__ Raw<SRC> zero_raw() {
  Raw<SRC> r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(r.q) / 16); ++i) r.q[i] = i32x4{0, 0, 0, 0};
  return r;
}

template <int SRC>
__device__ __forceinline__ typename Family<SRC>::Op to_op(const Raw<SRC>& r);

template <>
__device__ __forceinline__ OpBF to_op<DT_BF16>(const Raw<DT_BF16>& r) {
  OpBF o;
  o.v[0] = as_bf16x8(r.q[0]);
  o.v[1] = as_bf16x8(r.q[1]);
  return o;
}
template <>
__device__ __forceinline__ OpBF to_op<DT_F32>(const Raw<DT_F32>& r) {
  OpBF o;
  o.v[0] = as_bf16x8(pack_bf16x8(r.q[0], r.q[1]));
  o.v[1] = as_bf16x8(pack_bf16x8(r.q[2], r.q[3]));
  return o;
}
template <>
__device__ __forceinline__ OpF8 to_op<DT_E4M3>(const Raw<DT_E4M3>& r) {
  OpF8 o;
  o.v = i32x8{r.q[0][0], r.q[0][1], r.q[0][2], r.q[0][3],
              r.q[1][0], r.q[1][1], r.q[1][2], r.q[1][3]};
  return o;
}

__device__ __forceinline__ f32x4 mma(const OpBF& a, const OpBF& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[0], b.v[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[1], b.v[1], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ f32x4 mma(const OpF8& a, const OpF8& b, f32x4 c) {
  // format code 0 = E4M3 for both operands; zero scale operands select the
  // unscaled v_mfma_f32_16x16x128_f8f6f4.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a.v, b.v, c, 0, 0, 0, 0, 0, 0);
}

// SiLU(z) = z / (1 + e^-z) with the hardware base-2 exponential and
// reciprocal (each within about 1 ulp), so a few ulps from the rounded fp32
// value: z * rcp(1 + 2^(-z log2 e)).  Large negative z gives 2^(+big) = inf
// and z * rcp(inf) = -0, the limit.
__device__ __forceinline__ float silu(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.44269504088896340736f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace moe
