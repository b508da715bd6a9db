// route.hip -- top-k routing: one wave64 per token row.
//
// Dynamic token -> expert routing with k experts per token is the first stage
// of the fused op ("Amazon SageMaker AI 上的 Mixture-of-Experts 内核工程优化",
// introduction; topk = 8 in uniquestudio's digest, "背景与事实").  The pages
// give no selection rule; this kernel takes the k largest fp32 logits
// (descending, equal values to the lower expert id) and softmax weights.
//
// Each lane holds the logits of experts lane, lane+64, ... in registers.  A
// selection round is a lane-local best followed by a 6-step xor-shuffle
// reduction on (value, id); the winning lane marks its entry taken.  Weights
// are computed in fp32 from exp(l - l_max), l_max being the first winner.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

template <int NPER>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int M, int E, int k, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* l = logits + (size_t)row * E;

  float v[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    int e = lane + kWave * i;
    v[i] = (e < E) ? l[e] : 0.0f;
  }
  unsigned taken = 0;
  float my_v = 0.0f;
  int my_id = 0;
  float lmax = 0.0f;

  for (int j = 0; j < k; ++j) {
    // lane-local best: ids increase with i, so a strict '>' keeps the lower id
    float bv = 0.0f;
    int bid = -1;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      int e = lane + kWave * i;
      bool ok = (e < E) && !((taken >> i) & 1u);
      if (ok && (bid < 0 || v[i] > bv)) {
        bv = v[i];
        bid = e;
      }
    }
    // wave reduction on (value desc, id asc); bid < 0 marks "nothing left"
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o, kWave);
      int oid = __shfl_xor(bid, o, kWave);
      bool take = oid >= 0 && (bid < 0 || ov > bv || (ov == bv && oid < bid));
      if (take) {
        bv = ov;
        bid = oid;
      }
    }
    if ((bid & 63) == lane) taken |= 1u << (bid >> 6);
    if (j == 0) lmax = bv;
    if (lane == j) {
      my_v = bv;
      my_id = bid;
    }
  }

  float p = (lane < k) ? expf(my_v - lmax) : 0.0f;
  float z;
  if (renorm) {
    z = wave_sum(p);
  } else {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (lane + kWave * i < E) s += expf(v[i] - lmax);
    z = wave_sum(s);
  }
  if (lane < k) {
    ids[(size_t)row * k + lane] = my_id;
    wts[(size_t)row * k + lane] = p / z;
  }
}

int launch_route_topk(const float* logits, int M, int E, int k, int renorm,
                      int32_t* ids, float* wts, hipStream_t stream) {
  if (M == 0) return 0;
  dim3 grid((M + 3) / 4), block(256);
  int nper = (E + kWave - 1) / kWave;
#define ROUTE_CASE(N)                                                          \
  if (nper <= N) {                                                             \
    hipLaunchKernelGGL(route_topk_kernel<N>, grid, block, 0, stream, logits, M, \
                       E, k, renorm, ids, wts);                                \
    return (int)hipGetLastError();                                             \
  }
  ROUTE_CASE(1)
  ROUTE_CASE(2)
  ROUTE_CASE(4)
  ROUTE_CASE(8)
  ROUTE_CASE(16)
#undef ROUTE_CASE
  return -1;
}

}  // namespace moe
