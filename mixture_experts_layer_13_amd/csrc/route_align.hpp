// route_align.hpp -- device bodies of top-k routing (one wave per token row)
// and of the per-expert alignment of one 1024-pair chunk; used by the
// separate route / align kernels and by the fused one-workgroup kernel.
//
// Routing: "Amazon SageMaker AI 上的 Mixture-of-Experts 内核工程优化",
// introduction (token routing); k experts per token, uniquestudio digest,
// "背景与事实".  Alignment: the same post, "Backend routing for FP8 tensor
// quantization" (variable token bucketing onto the active experts).
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kChunk = 1024;                 // pairs per alignment chunk / threads
constexpr int kChunkWaves = kChunk / kWave;  // 16

// Order-preserving unsigned key of a binary32 value (-0 and +0 map to the
// same key, as they compare equal).
__device__ __forceinline__ uint32_t float_key(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);  // -0 + 0 = +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k of one token's logits: lanes 0..k-1 return the j-th selected id
// (descending logit, equal values to the lower id) and its fp32 softmax
// weight (over all E, or renormalised over the k selected).  Lane `lane`
// holds the logits of experts lane, lane + 64, ... in vin[] (entries past E
// are ignored).  Selection is a radix select on the order-preserving keys
// with ballots (32 bit steps, no data exchange between lanes); the k winners
// are then ranked by (key desc, id asc) with one broadcast per winner.  Must
// be called by a whole wave.
template <int NPER>
__device__ __forceinline__ void route_values(const float (&vin)[NPER], int E, int k, int renorm,
                                             int lane, int& out_id, float& out_w) {
  float v[NPER];
  uint32_t key[NPER];
  uint64_t cur[NPER], sel[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + kWave * i;
    v[i] = (e < E) ? vin[i] : 0.0f;
    key[i] = float_key(v[i]);
    cur[i] = __ballot(e < E);
    sel[i] = 0;
  }
  // radix select of the k largest keys: `cur` = undecided candidates that
  // share the current key prefix, `sel` = certainly selected
  int need = k;
  for (int b = 31; b >= 0 && need > 0; --b) {
    uint64_t ones[NPER];
    int c = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      ones[i] = cur[i] & __ballot((key[i] >> b) & 1u);
      c += __popcll(ones[i]);
    }
    if (c >= need) {
#pragma unroll
      for (int i = 0; i < NPER; ++i) cur[i] = ones[i];
    } else {
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        sel[i] |= ones[i];
        cur[i] &= ~ones[i];
      }
      need -= c;
    }
    // every candidate left ranks above every key outside sel and cur: when
    // exactly `need` are left they are the rest of the k
    int left = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) left += __popcll(cur[i]);
    if (left == need) {
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        sel[i] |= cur[i];
        cur[i] = 0;
      }
      need = 0;
    }
  }
  // `cur` now holds equal keys: the lowest ids (i first, then lane) complete k
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    while (need > 0 && cur[i]) {
      const uint64_t lo = cur[i] & (~cur[i] + 1);
      sel[i] |= lo;
      cur[i] &= ~lo;
      --need;
    }
  }
  // rank of each winner = number of winners ahead of it in (key desc, id asc)
  int rank[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) rank[i] = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    uint64_t m = sel[i];
    while (m) {
      const int ln = __ffsll((long long)m) - 1;
      m &= m - 1;
      const uint32_t kk = (uint32_t)__builtin_amdgcn_readlane((int)key[i], ln);
      const int id = ln + kWave * i;
#pragma unroll
      for (int i2 = 0; i2 < NPER; ++i2) {
        const bool mine = (sel[i2] >> lane) & 1ull;
        const int my_id = lane + kWave * i2;
        if (mine && (kk > key[i2] || (kk == key[i2] && id < my_id))) ++rank[i2];
      }
    }
  }
  // deliver in rank order: winner j goes to lane j; weights in fp32
  float lmax = 0.0f, zsel = 0.0f, my_p = 0.0f;
  out_id = 0;
  for (int j = 0; j < k; ++j) {
    bool has = false;
    float mv = 0.0f;
    int mid = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (((sel[i] >> lane) & 1ull) && rank[i] == j) {
        has = true;
        mv = v[i];
        mid = lane + kWave * i;
      }
    const int ln = __ffsll((long long)__ballot(has)) - 1;
    const float vv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mv), ln));
    const int id = __builtin_amdgcn_readlane(mid, ln);
    if (j == 0) lmax = vv;
    const float p = expf(vv - lmax);
    zsel += p;
    if (lane == j) {
      out_id = id;
      my_p = p;
    }
  }
  float z = zsel;
  if (!renorm) {
    float s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (lane + kWave * i < E) s2 += expf(v[i] - lmax);
    z = wave_sum(s2);
  }
  out_w = my_p / z;
}

// route_values on the logits row l[0:E) in memory.
template <int NPER>
__device__ __forceinline__ void route_row(const float* __restrict__ l, int E, int k, int renorm,
                                          int lane, int& out_id, float& out_w) {
  float v[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + kWave * i;
    v[i] = (e < E) ? l[e] : 0.0f;
  }
  route_values<NPER>(v, E, k, renorm, lane, out_id, out_w);
}

// Exclusive scan of v over a kChunk-thread workgroup; returns the prefix for
// this thread and the total in *total.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
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

// Alignment of chunk c (pairs [c*1024, c*1024+1024)) by a 1024-thread
// workgroup.  With nchunks == 1 the chunk counts itself; otherwise hist
// [E][nchunks] holds every chunk's counts.  Deterministic: LDS atomics only
// count, positions come from prefix sums and ballot ranks.
// sm: LDS of (3E + 2 + 16(E+1) + 16) ints.
__device__ __forceinline__ void align_chunk(
    const int32_t* ids, int P, int E, int bm, int nchunks, int c,
    const int32_t* __restrict__ hist, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ offsets_out,
    int32_t* __restrict__ pair_pos, int32_t* __restrict__ num_padded, int32_t* sm) {
  int32_t* total = sm;                       // [E]
  int32_t* base = total + E;                 // [E]
  int32_t* off = base + E;                   // [E+1]
  int32_t* s_total = off + (E + 1);          // [1]
  int32_t* wcnt = s_total + 1;               // [16][E+1]
  int32_t* wsum = wcnt + kChunkWaves * (E + 1);  // [16]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // 1. totals per expert and this chunk's base per expert
  if (nchunks == 1) {
    for (int e = tid; e < E; e += kChunk) {
      total[e] = 0;
      base[e] = 0;
    }
    __syncthreads();
    if (tid < P) {
      int id = ids[tid];
      if (id >= 0 && id < E) atomicAdd(&total[id], 1);
    }
  } else {
    // one wave per expert, its lanes over the chunks (hist is [E][nchunks])
    for (int e = w; e < E; e += kChunkWaves) {
      int t = 0, b = 0;
      for (int cc = lane; cc < nchunks; cc += kWave) {
        const int h = hist[(size_t)e * nchunks + cc];
        if (cc < c) b += h;
        t += h;
      }
      t = wave_sum_i(t);
      b = wave_sum_i(b);
      if (lane == 0) {
        total[e] = t;
        base[e] = b;
      }
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
    *s_total = tot;
  }
  __syncthreads();
  if (c == 0) {
    for (int e = tid; e <= E; e += kChunk) offsets_out[e] = off[e];
    if (tid == 0) *num_padded = *s_total;
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

}  // namespace moe
