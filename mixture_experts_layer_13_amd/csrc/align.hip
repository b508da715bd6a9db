// align.hip -- per-expert token bucketing: a stable counting sort of the
// P = M*topk flat pair indices by expert id, each expert segment padded to a
// multiple of block_m.  This gives the grouped GEMMs expert-contiguous,
// tile-padded token blocks, the "variable token bucketing" that maps small,
// fragmented token groups onto the active experts' weights in
// "Amazon SageMaker AI 上的 Mixture-of-Experts 内核工程优化", section "Backend
// routing for FP8 tensor quantization".
//
// Deterministic by construction: LDS atomics only count, and every position
// comes from prefix sums plus a rank computed with ballots, so no output
// depends on the order in which atomics land.
//
//   chunk c = pairs [c*1024, (c+1)*1024), one 1024-thread workgroup each.
//   hist kernel (only when there is more than one chunk): counts per chunk,
//     stored expert-major.
//   scatter kernel: totals and the chunk's base per expert from the counts
//     (one wave per expert, its lanes across the chunks),
//     padded offsets by a block scan, the in-chunk rank of each pair among
//     equal ids (11-bit ballot match inside a wave + per-wave counts in LDS),
//     then the writes; padding sentinels and block->expert entries are
//     spread over the chunks' waves.
#include "common.hpp"
#include "launch.hpp"
#include "route_align.hpp"

namespace moe {


__global__ __launch_bounds__(kChunk) void align_hist_kernel(
    const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ hist) {
  extern __shared__ int32_t cnt[];  // [E]
  for (int e = threadIdx.x; e < E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  int f = blockIdx.x * kChunk + threadIdx.x;
  if (f < P) {
    int id = ids[f];
    if (id >= 0 && id < E) atomicAdd(&cnt[id], 1);
  }
  __syncthreads();
  // expert-major [E][nchunks]: a scatter workgroup reads one expert's counts
  // of all chunks as one contiguous run
  for (int e = threadIdx.x; e < E; e += kChunk)
    hist[(size_t)e * gridDim.x + blockIdx.x] = cnt[e];
}

__global__ __launch_bounds__(kChunk) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, int bm, int nchunks,
    const int32_t* __restrict__ hist, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ offsets_out,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ num_padded) {
  extern __shared__ int32_t sm[];
  align_chunk(ids, P, E, bm, nchunks, blockIdx.x, hist, sorted_ids, block_expert, offsets_out,
              pair_pos, num_padded, sm);
}

// Routing and alignment in one workgroup when all pairs fit one chunk (the
// decode case): the ids stay in LDS between the two phases.
template <int NPER>
__global__ __launch_bounds__(kChunk) void route_align_kernel(
    const float* __restrict__ logits, int M, int E, int k, int renorm, int bm,
    int32_t* __restrict__ ids, float* __restrict__ wts, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ offsets_out,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ num_padded) {
  extern __shared__ int32_t sm[];
  int32_t* lids = sm;             // [kChunk]
  int32_t* scratch = sm + kChunk;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int row = w; row < M; row += kChunkWaves) {
    int id;
    float wt;
    route_row<NPER>(logits + (size_t)row * E, E, k, renorm, lane, id, wt);
    if (lane < k) {
      ids[(size_t)row * k + lane] = id;
      wts[(size_t)row * k + lane] = wt;
      lids[row * k + lane] = id;
    }
  }
  __syncthreads();
  align_chunk(lids, M * k, E, bm, 1, 0, nullptr, sorted_ids, block_expert, offsets_out, pair_pos,
              num_padded, scratch);
}

static size_t align_lds_bytes(int E);

size_t align_workspace_bytes(int M, int topk, int E) {
  long long P = (long long)M * topk;
  long long nch = (P + kChunk - 1) / kChunk;
  return nch > 1 ? (size_t)(nch * E * 4) : 0;
}

int launch_align(const int32_t* ids, int M, int topk, int E, int bm,
                 int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                 int32_t* pair_pos, int32_t* num_padded, void* ws,
                 hipStream_t stream) {
  int P = M * topk;
  int nch = (P + kChunk - 1) / kChunk;
  if (nch < 1) nch = 1;
  int32_t* hist = reinterpret_cast<int32_t*>(ws);
  if (nch > 1) {
    hipLaunchKernelGGL(align_hist_kernel, dim3(nch), dim3(kChunk), E * 4, stream,
                       ids, P, E, hist);
    int err = (int)hipGetLastError();
    if (err) return err;
  }
  size_t lds = align_lds_bytes(E);
  static OncePerDevice attr;  // E = 1024 needs ~78 KiB of the 160 KiB LDS
  int err = attr.run([] {
    return (int)hipFuncSetAttribute((const void*)align_scatter_kernel,
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)align_lds_bytes(1024));
  });
  if (err) return err;
  hipLaunchKernelGGL(align_scatter_kernel, dim3(nch), dim3(kChunk), lds, stream,
                     ids, P, E, bm, nch, hist, sorted_ids, block_expert, offsets,
                     pair_pos, num_padded);
  return (int)hipGetLastError();
}

static size_t align_lds_bytes(int E) {
  return (size_t)(3 * E + 2 + kChunkWaves * (E + 1) + kChunkWaves) * 4;
}

int launch_route_align(const float* logits, int M, int E, int k, int renorm, int bm,
                       int32_t* ids, float* wts, int32_t* sorted_ids, int32_t* block_expert,
                       int32_t* offsets, int32_t* pair_pos, int32_t* num_padded,
                       hipStream_t stream) {
  const size_t lds = (size_t)kChunk * 4 + align_lds_bytes(E);
  const int nper = (E + kWave - 1) / kWave;
#define RA_CASE(N)                                                                      \
  if (nper <= N) {                                                                      \
    static OncePerDevice attr;                                                          \
    int err = attr.run([] {                                                             \
      return (int)hipFuncSetAttribute((const void*)route_align_kernel<N>,               \
                                      hipFuncAttributeMaxDynamicSharedMemorySize,       \
                                      (int)(kChunk * 4 + align_lds_bytes(1024)));       \
    });                                                                                 \
    if (err) return err;                                                                \
    hipLaunchKernelGGL(route_align_kernel<N>, dim3(1), dim3(kChunk), lds, stream, logits, \
                       M, E, k, renorm, bm, ids, wts, sorted_ids, block_expert, offsets, \
                       pair_pos, num_padded);                                           \
    return (int)hipGetLastError();                                                      \
  }
  RA_CASE(1)
  RA_CASE(2)
  RA_CASE(4)
  RA_CASE(8)
  RA_CASE(16)
#undef RA_CASE
  return -1;
}

}  // namespace moe
