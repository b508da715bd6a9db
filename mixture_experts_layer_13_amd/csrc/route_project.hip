// route_project.hip -- token routing from the hidden states: a linear router
// projection (logits = x . W_r^T, one weight row per expert) followed by the
// top-k routing of route.hip.
//
// Token routing is the first stage the fused op takes over ("Amazon
// SageMaker AI 上的 Mixture-of-Experts 内核工程优化", introduction); the pages
// give no router formula, and the layer reads it as a linear router whose
// weight W_r [E, K] is stored like the expert weights (the hidden dimension
// contiguous).
//
// Two launches.  The projection is split over K so that the whole chip
// streams W_r: a workgroup (4 waves) computes a 64-token x 64-expert tile of
// one K slice on v_mfma_f32_16x16x32_bf16 (router rows on the row operand,
// tokens on the column operand, fp32 accumulation; f32 inputs are rounded to
// bf16 on load, as the f32 expert path does) and stores its partial sums.
// Each wave takes the whole tile over every fourth K step (x and W_r of the
// tile are read once; with a wave per 16 experts x was read four times and
// 8192 tokens' projection took 44.6 us instead of 28.5).
// The second launch adds a token's slices in a fixed order (so results do
// not depend on scheduling), keeps the logits in registers and routes them
// with the selection and weights of moe_route_topk.  (A single launch that
// routes inside the projection's workgroups has to bring every expert's
// logit of a token into one workgroup, which then streams all of W_r
// through one CU: measured 25 us for one token and 4096 x 64 bf16 weights,
// against a few us here.)
#include "common.hpp"
#include "launch.hpp"
#include "route_align.hpp"

namespace moe {

constexpr int kRpNt = 4;                // 16-row MFMA blocks per tile side
constexpr int kRpTok = 16 * kRpNt;      // token rows per projection workgroup
constexpr int kRpExp = 16 * kRpNt;      // experts per projection workgroup
constexpr int kRpTargetWg = 1024;       // projection workgroups the K split aims at
constexpr int kRpSumBatch = 8;          // partial sums loaded together by the reduction

typedef __bf16 rp_bf16x8 __attribute__((ext_vector_type(8)));

// Number of K slices: the largest divisor of K / 128 that keeps the
// projection grid at or under kRpTargetWg workgroups (1 when the token and
// expert tiles alone fill it).
int route_project_slices(int M, int K, int E) {
  const long long base = (long long)((M + kRpTok - 1) / kRpTok) * ((E + kRpExp - 1) / kRpExp);
  const int kc = K / 128;
  int s = 1;
  for (int d = 1; d <= kc; ++d)
    if (kc % d == 0 && base * d <= kRpTargetWg) s = d;
  return s;
}

size_t route_project_workspace_bytes(int M, int K, int E) {
  return (size_t)route_project_slices(M, K, E) * (size_t)M * (size_t)E * sizeof(float);
}

// Eight consecutive values of a row as bf16 bits (4 dwords): bf16 as stored,
// f32 rounded to nearest even.
template <int T>
__device__ __forceinline__ i32x4 rp_load8(const void* base, size_t idx) {
  if constexpr (T == DT_BF16) {
    return ld16(reinterpret_cast<const uint16_t*>(base) + idx);
  } else {
    const float* p = reinterpret_cast<const float*>(base) + idx;
    const i32x4 a = ld16(p), b = ld16(p + 4);
    return i32x4{(int)pack_bf16x2(__int_as_float(a[0]), __int_as_float(a[1])),
                 (int)pack_bf16x2(__int_as_float(a[2]), __int_as_float(a[3])),
                 (int)pack_bf16x2(__int_as_float(b[0]), __int_as_float(b[1])),
                 (int)pack_bf16x2(__int_as_float(b[2]), __int_as_float(b[3]))};
  }
}

__device__ __forceinline__ f32x4 rp_mma(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(rp_bf16x8, a),
                                                 __builtin_bit_cast(rp_bf16x8, b), c, 0, 0, 0);
}

// grid (blocks of 64 tokens, blocks of 64 experts, K slices of kslice
// values): part[slice][t][e] = sum over the slice of x[t, k] * wr[e, k].
// Every wave computes the whole 64 x 64 tile (4 x 4 MFMA blocks: four
// router-row loads and four token loads feed 16 MFMAs per K step) over every
// fourth K step of the slice, so the tile's x and W_r are each read once;
// the four waves' sums are then added in LDS in wave order.
template <int T>
__global__ __launch_bounds__(256) void route_project_partial_kernel(
    const void* __restrict__ x, const void* __restrict__ wr, int M, int K, int E, int kslice,
    float* __restrict__ part) {
  __shared__ f32x4 red[3][kRpNt * kRpNt][kWave];  // waves 1-3, 48 KiB
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int s = blockIdx.z;
  const int t0 = blockIdx.x * kRpTok, e0 = blockIdx.y * kRpExp;
  // rows past M or E read row 0; their sums are not stored
  const size_t k0 = (size_t)s * kslice + g * 8;
  size_t xoff[kRpNt], woff[kRpNt];
#pragma unroll
  for (int j = 0; j < kRpNt; ++j) {
    const int tok = t0 + 16 * j + r16, e = e0 + 16 * j + r16;
    xoff[j] = (size_t)(tok < M ? tok : 0) * K + k0;
    woff[j] = (size_t)(e < E ? e : 0) * K + k0;
  }
  const int nks = kslice / 32;  // a multiple of 4: every wave takes nks / 4 steps
  f32x4 acc[kRpNt][kRpNt];      // [token block][expert block]
#pragma unroll
  for (int j = 0; j < kRpNt; ++j)
#pragma unroll
    for (int i = 0; i < kRpNt; ++i) acc[j][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int st = wv; st < nks; st += 4) {
    i32x4 A[kRpNt], B[kRpNt];
#pragma unroll
    for (int j = 0; j < kRpNt; ++j) {
      A[j] = rp_load8<T>(wr, woff[j] + (size_t)st * 32);
      B[j] = rp_load8<T>(x, xoff[j] + (size_t)st * 32);
    }
#pragma unroll
    for (int j = 0; j < kRpNt; ++j)
#pragma unroll
      for (int i = 0; i < kRpNt; ++i) acc[j][i] = rp_mma(A[i], B[j], acc[j][i]);
  }
  if (wv > 0) {
#pragma unroll
    for (int j = 0; j < kRpNt; ++j)
#pragma unroll
      for (int i = 0; i < kRpNt; ++i) red[wv - 1][j * kRpNt + i][lane] = acc[j][i];
  }
  __syncthreads();
  if (wv != 0) return;
  // lane holds experts e0 + 16 i + 4g + q of tokens t0 + 16 j + r16
#pragma unroll
  for (int j = 0; j < kRpNt; ++j) {
    const int tok = t0 + 16 * j + r16;
#pragma unroll
    for (int i = 0; i < kRpNt; ++i) {
      f32x4 v = acc[j][i];
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        const f32x4 p = red[w][j * kRpNt + i][lane];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += p[q];
      }
      if (tok < M) {
        float* dst = part + ((size_t)s * M + tok) * E;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ee = e0 + 16 * i + 4 * g + q;
          if (ee < E) dst[ee] = v[q];
        }
      }
    }
  }
}

// One wave per token: logits = the slices' sums in slice order, then the
// routing of moe_route_topk.
template <int NPER>
__global__ __launch_bounds__(256) void route_project_reduce_kernel(
    const float* __restrict__ part, int S, int M, int E, int k, int renorm,
    float* __restrict__ logits_out, int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  float v[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + kWave * i;
    float sum = 0.0f;
    if (e < E) {
      const float* p = part + (size_t)row * E + e;
      const size_t slice = (size_t)M * E;
      for (int s0 = 0; s0 < S; s0 += kRpSumBatch) {  // loads in flight together, sums in order
        float t[kRpSumBatch];
#pragma unroll
        for (int u = 0; u < kRpSumBatch; ++u) t[u] = s0 + u < S ? p[(size_t)(s0 + u) * slice] : 0.0f;
#pragma unroll
        for (int u = 0; u < kRpSumBatch; ++u)
          if (s0 + u < S) sum += t[u];
      }
      if (logits_out) logits_out[(size_t)row * E + e] = sum;
    }
    v[i] = sum;
  }
  int id;
  float w;
  route_values<NPER>(v, E, k, renorm, lane, id, w);
  if (lane < k) {
    ids[(size_t)row * k + lane] = id;
    wts[(size_t)row * k + lane] = w;
  }
}

template <int NPER>
static void rp_reduce(const float* part, int S, int M, int E, int k, int renorm, float* logits,
                      int32_t* ids, float* wts, hipStream_t st) {
  hipLaunchKernelGGL((route_project_reduce_kernel<NPER>), dim3((M + 3) / 4), dim3(256), 0, st, part,
                     S, M, E, k, renorm, logits, ids, wts);
}

int launch_route_project(const void* x, const void* wr, int dtype, int M, int K, int E, int k,
                         int renorm, float* logits, int32_t* ids, float* wts, void* ws,
                         hipStream_t st) {
  if (M == 0) return 0;
  const int S = route_project_slices(M, K, E);
  float* part = reinterpret_cast<float*>(ws);
  const dim3 grid((M + kRpTok - 1) / kRpTok, (E + kRpExp - 1) / kRpExp, S);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(route_project_partial_kernel<DT_BF16>, grid, dim3(256), 0, st, x, wr, M, K,
                       E, K / S, part);
  else
    hipLaunchKernelGGL(route_project_partial_kernel<DT_F32>, grid, dim3(256), 0, st, x, wr, M, K, E,
                       K / S, part);
  int err = (int)hipGetLastError();
  if (err) return err;
  const int nper = (E + kWave - 1) / kWave;
  if (nper <= 1)
    rp_reduce<1>(part, S, M, E, k, renorm, logits, ids, wts, st);
  else if (nper <= 2)
    rp_reduce<2>(part, S, M, E, k, renorm, logits, ids, wts, st);
  else if (nper <= 4)
    rp_reduce<4>(part, S, M, E, k, renorm, logits, ids, wts, st);
  else if (nper <= 8)
    rp_reduce<8>(part, S, M, E, k, renorm, logits, ids, wts, st);
  else if (nper <= 16)
    rp_reduce<16>(part, S, M, E, k, renorm, logits, ids, wts, st);
  else
    return -1;
  return (int)hipGetLastError();
}

}  // namespace moe
