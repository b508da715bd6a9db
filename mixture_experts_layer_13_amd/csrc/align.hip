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
//   hist kernel (only when there is more than one chunk): counts per chunk.
//   scatter kernel: totals and the chunk's base per expert from the counts,
//     padded offsets by a block scan, the in-chunk rank of each pair among
//     equal ids (11-bit ballot match inside a wave + per-wave counts in LDS),
//     then the writes; padding sentinels and block->expert entries are
//     spread over the chunks' waves.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kChunk = 1024;
constexpr int kChunkWaves = kChunk / kWave;  // 16

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
  for (int e = threadIdx.x; e < E; e += kChunk)
    hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Exclusive scan of v over the whole workgroup (kChunk threads); returns the
// prefix for this thread and writes the total to *total.
__device__ int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    int s = (lane < kChunkWaves) ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(s, o, kWave);
      if (lane >= o) s += y;
    }
    if (lane < kChunkWaves) wsum[lane] = s;  // inclusive per wave
  }
  __syncthreads();
  int before = (w == 0) ? 0 : wsum[w - 1];
  *total = wsum[kChunkWaves - 1];
  int r = before + x - v;
  __syncthreads();  // wsum may be reused by the caller
  return r;
}

__global__ __launch_bounds__(kChunk) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, int bm, int nchunks,
    const int32_t* __restrict__ hist, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ offsets_out,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ num_padded) {
  // LDS: total[E], base[E], off[E+1], wcnt[16][E+1], wsum[16]
  extern __shared__ int32_t sm[];
  int32_t* total = sm;
  int32_t* base = total + E;
  int32_t* off = base + E;
  int32_t* wcnt = off + (E + 1);
  int32_t* wsum = wcnt + kChunkWaves * (E + 1);
  __shared__ int32_t s_total;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = blockIdx.x;

  // 1. totals per expert and this chunk's base per expert
  if (nchunks == 1) {
    for (int e = tid; e < E; e += kChunk) {
      total[e] = 0;
      base[e] = 0;
    }
    __syncthreads();
    int f = tid;
    if (f < P) {
      int id = ids[f];
      if (id >= 0 && id < E) atomicAdd(&total[id], 1);
    }
  } else {
    for (int e = tid; e < E; e += kChunk) {
      int t = 0, b = 0;
      for (int cc = 0; cc < nchunks; ++cc) {
        int h = hist[(size_t)cc * E + e];
        if (cc < c) b += h;
        t += h;
      }
      total[e] = t;
      base[e] = b;
    }
  }
  for (int i = tid; i < kChunkWaves * (E + 1); i += kChunk) wcnt[i] = 0;
  __syncthreads();

  // 2. padded offsets (E <= 1024 = one value per thread)
  int q = 0;
  if (tid < E) q = (total[tid] + bm - 1) / bm * bm;
  int tot;
  int pre = block_excl_scan(q, wsum, &tot);
  if (tid < E) off[tid] = pre;
  if (tid == 0) {
    off[E] = tot;
    s_total = tot;
  }
  __syncthreads();
  if (c == 0) {
    for (int e = tid; e <= E; e += kChunk) offsets_out[e] = off[e];
    if (tid == 0) *num_padded = s_total;
  }

  // 3. in-chunk rank among equal ids (ids outside [0,E) get key E: dropped)
  const int f = c * kChunk + tid;
  int key = 2047;  // lanes past P: a key no real pair has
  if (f < P) {
    int id = ids[f];
    key = (id >= 0 && id < E) ? id : E;
  }
  uint64_t match = ~0ull;
#pragma unroll
  for (int b = 0; b < 11; ++b) {
    uint64_t bal = __ballot((key >> b) & 1);
    match &= ((key >> b) & 1) ? bal : ~bal;
  }
  const int in_wave = __popcll(match & lanemask_lt(lane));
  const bool leader = in_wave == 0;
  if (leader && key <= E) wcnt[w * (E + 1) + key] = __popcll(match);
  __syncthreads();
  if (f < P) {
    if (key < E) {
      int r = in_wave;
      for (int ww = 0; ww < w; ++ww) r += wcnt[ww * (E + 1) + key];
      int pos = off[key] + base[key] + r;
      sorted_ids[pos] = f;
      pair_pos[f] = pos;
    } else {
      pair_pos[f] = -1;
    }
  }

  // 4. padding sentinels and block -> expert map; expert e is handled by
  //    global wave (e mod (nchunks*16)).
  const int gw = c * kChunkWaves + w, nw = nchunks * kChunkWaves;
  for (int e = gw; e < E; e += nw) {
    int s0 = off[e] + total[e], s1 = off[e + 1];
    for (int s = s0 + lane; s < s1; s += kWave) sorted_ids[s] = P;
    for (int b = off[e] / bm + lane; b < s1 / bm; b += kWave) block_expert[b] = e;
  }
}

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
  size_t lds = (size_t)(3 * E + 1 + kChunkWaves * (E + 1) + kChunkWaves) * 4;
  static bool attr_set = false;  // E = 1024 needs ~78 KiB of the 160 KiB LDS
  if (!attr_set) {
    int err = (int)hipFuncSetAttribute((const void*)align_scatter_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)((3 * 1024 + 1 + kChunkWaves * 1025 + kChunkWaves) * 4));
    if (err) return err;
    attr_set = true;
  }
  hipLaunchKernelGGL(align_scatter_kernel, dim3(nch), dim3(kChunk), lds, stream,
                     ids, P, E, bm, nch, hist, sorted_ids, block_expert, offsets,
                     pair_pos, num_padded);
  return (int)hipGetLastError();
}

}  // namespace moe
