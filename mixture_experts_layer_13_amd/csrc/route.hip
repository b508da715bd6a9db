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
#include "route_align.hpp"

namespace moe {

template <int NPER>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int M, int E, int k, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  int id;
  float w;
  route_row<NPER>(logits + (size_t)row * E, E, k, renorm, lane, id, w);
  if (lane < k) {
    ids[(size_t)row * k + lane] = id;
    wts[(size_t)row * k + lane] = w;
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
