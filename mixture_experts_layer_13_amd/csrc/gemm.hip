// gemm.hip -- grouped expert GEMMs of the fused MoE layer on gfx950 MFMA.
//
// Pages cited:
//   [post] "Amazon SageMaker AI 上的 Mixture-of-Experts 内核工程优化" (English
//          text of the AWS Machine Learning Blog post);
//   [faq]  uniquestudio AI-news digest of the same post, "背景与事实".
//
// The expert product is A[M,K] x B[K,N] with M token rows ([post], "Swap-AB
// for WGMMA utilization").  On Hopper the post moves the wide expert
// dimension into the operand slot whose tile height is fixed at 64 by
// computing B^T x A^T ([faq]).  CDNA4's MFMA tiles are 16 wide on both sides,
// so what carries over to gfx950 is the memory side of that idea: expert
// weight rows (K-contiguous B^T rows) sit on the MFMA row operand and are
// streamed straight from HBM into registers, each lane reading 32 contiguous
// bytes per step, while the few tokens of a decode batch occupy the 16-wide
// column operand.  Every kernel here computes C^T = W x X^T.
//
// The post's FP8 path keeps tensor scaling, the matmul and the expert
// aggregation in one pass over HBM ([post], "Backend routing for FP8 tensor
// quantization"); here the dequant scales, SiLU * up and the routing weight
// are applied to the fp32 accumulators in registers.
//
// The bf16 and E4M3 decode products run on the expert rings (ring.hip) and
// the large-batch ones on the tiles of prefill.hip / prefill2.hip.  This file
// holds the rest, chosen on the host:
//   stream (M <= 64 where the rings do not apply -- f32 weights, or weight
//     rows that are not whole 512-byte ring stages -- and the down product
//     below 4 tokens): gate/up kernel over (16-row tile, active expert) with
//     the K loop split across 4 waves; down kernel per 16 output rows that
//     walks every active expert and keeps the weighted top-k combine in LDS.
//   tile (M > 64 with f32 weights or token blocks under 128 rows): one
//     workgroup per (64-row weight tile, block_m token block of one expert);
//     token rows staged in LDS and shared by 4 waves; the down-projection
//     rows go to y, which the combine kernel sums with the routing weights.
//   combine: out[t] = sum over the top-k slots of w[t, j] * y[pair row].
#include "common.hpp"
#include "launch.hpp"

namespace moe {

template <int T>
constexpr int fam_step() {
  return 4 * Family<T>::kPerLane;  // K per step
}
template <int T>
constexpr int lane_bytes() {
  return Family<T>::kPerLane * Family<T>::kBytes;  // bytes per lane per step
}


template <int OT>
__device__ __forceinline__ void store_out4(void* out, size_t idx, const float v[4]);

// ======================================================== stream: gate/up
//
// The K loop of both stream kernels is software-pipelined in registers: a
// wave holds two groups of U steps and issues the loads of the next group
// before the MFMAs of the current one, so about 2U steps of weight rows stay
// in flight per wave without waiting on the arithmetic.

constexpr int kG1Waves = 4;
constexpr int kG1Unroll1 = 2;      // K steps per group, one 16-token column block
constexpr int kG1Unroll2 = 1;      // K steps per group, two column blocks
constexpr int kG2Unroll1 = 2;      // down GEMM, one column block
constexpr int kG2Unroll2 = 2;      // down GEMM, two column blocks
constexpr int kStreamMaxNcb = 2;   // column blocks per pass (more tokens: more passes)
constexpr bool kNtWeights = false; // non-temporal expert-weight loads (slower here)

template <int SRC>
__device__ __forceinline__ Raw<SRC> load_w(const void* p) {
  if constexpr (kNtWeights) return load_raw_nt<SRC>(p);
  else return load_raw<SRC>(p);
}

template <int WT, int XT, int NCB, int U>
struct G1Group {
  Raw<WT> g[U], u[U];
  Raw<XT> x[U][NCB];
};

// Loads steps s, s + stride, ... (U of them, those below nsteps).
template <int WT, int XT, int NCB, int U>
__device__ __forceinline__ void g1_load(G1Group<WT, XT, NCB, U>& G, const char* wg,
                                        const char* wu, const char* const xr[NCB],
                                        const bool xv[NCB], int s, int stride, int nsteps,
                                        int ncb) {
  constexpr int SB_W = fam_step<WT>() * Family<WT>::kBytes;  // bytes per step (row)
  constexpr int SB_X = fam_step<XT>() * Family<XT>::kBytes;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int st = s + stride * u;
    if (st < nsteps) {
      G.g[u] = load_w<WT>(wg + (size_t)st * SB_W);
      G.u[u] = load_w<WT>(wu + (size_t)st * SB_W);
    }
  }
  // token rows past the expert's count contribute nothing: no load, zeros
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int st = s + stride * u;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      if (st < nsteps && cb < ncb)
        G.x[u][cb] = xv[cb] ? load_raw<XT>(xr[cb] + (size_t)st * SB_X) : zero_raw<XT>();
  }
}

template <int WT, int XT, int NCB, int U>
__device__ __forceinline__ void g1_mma(const G1Group<WT, XT, NCB, U>& G, int s, int stride,
                                       int nsteps, int ncb, f32x4 accg[NCB], f32x4 accu[NCB]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (s + stride * u < nsteps) {
      auto ag = to_op<WT>(G.g[u]);
      auto au = to_op<WT>(G.u[u]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        if (cb < ncb) {
          auto b = to_op<XT>(G.x[u][cb]);
          accg[cb] = mma(ag, b, accg[cb]);
          accu[cb] = mma(au, b, accu[cb]);
        }
      }
    }
  }
}

template <int WT, int XT, int NCB>
__global__ __launch_bounds__(256) void gemm1_stream_kernel(GemmArgs a) {
  constexpr int U = (NCB == 1) ? kG1Unroll1 : kG1Unroll2;
  __shared__ float red[kG1Waves][2][NCB][4][kWave];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;

  const int e = nth_active_expert(a.offsets, a.E, blockIdx.y);
  if (e < 0) return;  // uniform over the workgroup
  const int seg0 = a.offsets[e], seg1 = a.offsets[e + 1];
  const int me = segment_count(a.sorted_ids, seg0, seg1, a.P);
  const int n0 = blockIdx.x * 16;
  const int K = a.K, N = a.N;

  constexpr int WB = Family<WT>::kBytes, XB = Family<XT>::kBytes;
  const char* w13 = reinterpret_cast<const char*>(a.w13);
  const char* wg = w13 + (((size_t)e * 2 * N + n0 + r16) * K + (size_t)g * Family<WT>::kPerLane) * WB;
  const char* wu = wg + (size_t)N * K * WB;
  const char* xb = reinterpret_cast<const char*>(a.x) + (size_t)g * Family<XT>::kPerLane * XB;
  const int nsteps = K / fam_step<WT>();

  float scale = 1.0f;
  if (WT == DT_E4M3) scale = (*a.sx) * a.w13_scale[e];
  float hmax = 0.0f;

  for (int c0 = 0; c0 < me; c0 += 16 * NCB) {
    const int ncb = min(NCB, (me - c0 + 15) / 16);
    const char* xr[NCB];
    bool xv[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      int col = c0 + cb * 16 + r16;
      xv[cb] = col < me;
      int f = xv[cb] ? a.sorted_ids[seg0 + col] : a.sorted_ids[seg0];
      xr[cb] = xb + (size_t)(f / a.topk) * K * XB;
    }
    f32x4 accg[NCB], accu[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) accg[cb] = accu[cb] = f32x4{0, 0, 0, 0};

    {
      // wave wv takes steps wv, wv + 4, ...; groups of U steps, two in flight
      constexpr int S = kG1Waves * U;
      G1Group<WT, XT, NCB, U> A, B;
      int s = wv;
      g1_load(A, wg, wu, xr, xv, s, kG1Waves, nsteps, ncb);
      while (true) {
        if (s + S < nsteps) g1_load(B, wg, wu, xr, xv, s + S, kG1Waves, nsteps, ncb);
        g1_mma(A, s, kG1Waves, nsteps, ncb, accg, accu);
        s += S;
        if (s >= nsteps) break;
        if (s + S < nsteps) g1_load(A, wg, wu, xr, xv, s + S, kG1Waves, nsteps, ncb);
        g1_mma(B, s, kG1Waves, nsteps, ncb, accg, accu);
        s += S;
        if (s >= nsteps) break;
      }
    }

    // reduce the 4 K-slices
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red[wv][0][cb][i][lane] = accg[cb][i];
        red[wv][1][cb][i][lane] = accu[cb][i];
      }
    __syncthreads();
    // wave wv finishes column blocks cb = wv, wv + 4, ...
    for (int cb = wv; cb < ncb; cb += kG1Waves) {
      const int col = c0 + cb * 16 + r16;
      float h[4], g4[4], u4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int w = 0; w < kG1Waves; ++w) {
          gs += red[w][0][cb][i][lane];
          us += red[w][1][cb][i][lane];
        }
        g4[i] = gs * scale;
        u4[i] = us * scale;
        h[i] = silu(g4[i]) * u4[i];
      }
      if (a.probe) {
        if (col < me) probe_store(a, (size_t)(seg0 + col), n0 + 4 * g, g4, u4);
      } else if (col < me) {
        const size_t idx = (size_t)(seg0 + col) * N + n0 + 4 * g;
        if (WT == DT_E4M3) {
          st16(reinterpret_cast<float*>(a.h) + idx,
               i32x4{__float_as_int(h[0]), __float_as_int(h[1]), __float_as_int(h[2]),
                     __float_as_int(h[3])});
#pragma unroll
          for (int i = 0; i < 4; ++i) hmax = fmaxf(hmax, __builtin_fabsf(h[i]));
        } else {
          uint2 pk = make_uint2(pack_bf16x2(h[0], h[1]),
                                pack_bf16x2(h[2], h[3]));
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.h) + idx) = pk;
        }
      }
    }
    __syncthreads();
  }
  if (WT == DT_E4M3) {
    hmax = wave_max(hmax);
    if (lane == 0 && hmax > 0.0f) atomicMax(a.hmax_bits, __float_as_uint(hmax));
  }
}

// ============================================ stream: down + fused combine

constexpr int kG2Waves = 8;

template <int WT, int NCB, int U>
struct G2Group {
  static constexpr int HT = (WT == DT_E4M3) ? DT_E4M3 : DT_BF16;
  Raw<WT> w[U];
  Raw<HT> h[U][NCB];
};

template <int WT, int NCB, int U>
__device__ __forceinline__ void g2_load(G2Group<WT, NCB, U>& G, const char* wr,
                                        const char* const hr[NCB], const bool hv[NCB], int s,
                                        int nsteps, int ncb) {
  constexpr int HT = G2Group<WT, NCB, U>::HT;
  constexpr int SB_W = fam_step<WT>() * Family<WT>::kBytes;
  constexpr int SB_H = fam_step<HT>() * Family<HT>::kBytes;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (s + u < nsteps) G.w[u] = load_w<WT>(wr + (size_t)(s + u) * SB_W);
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      if (s + u < nsteps && cb < ncb)
        G.h[u][cb] = hv[cb] ? load_raw<HT>(hr[cb] + (size_t)(s + u) * SB_H) : zero_raw<HT>();
}

template <int WT, int NCB, int U>
__device__ __forceinline__ void g2_mma(const G2Group<WT, NCB, U>& G, int s, int nsteps, int ncb,
                                       f32x4 acc[NCB]) {
  constexpr int HT = G2Group<WT, NCB, U>::HT;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (s + u < nsteps) {
      auto aw = to_op<WT>(G.w[u]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        if (cb < ncb) acc[cb] = mma(aw, to_op<HT>(G.h[u][cb]), acc[cb]);
    }
  }
}

template <int WT, int OT, int NCB>
__global__ __launch_bounds__(512) void gemm2_stream_kernel(GemmArgs a) {
  constexpr int HT = (WT == DT_E4M3) ? DT_E4M3 : DT_BF16;
  constexpr int U = (NCB == 1) ? kG2Unroll1 : kG2Unroll2;
  extern __shared__ float acc_lds[];  // [kG2Waves][M][16]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int M = a.M, K = a.K, N = a.N;
  const int n0 = blockIdx.x * 16;

  for (int i = threadIdx.x; i < kG2Waves * M * 16; i += blockDim.x) acc_lds[i] = 0.0f;
  __syncthreads();
  float* my = acc_lds + (size_t)wv * M * 16;

  constexpr int WB = Family<WT>::kBytes, HB = Family<HT>::kBytes;
  const int nsteps = N / fam_step<WT>();
  const char* hbase = reinterpret_cast<const char*>(a.hq) + (size_t)g * Family<HT>::kPerLane * HB;

  int seen = 0;
  for (int base = 0; base < a.E; base += kWave) {
    const int ee = base + lane;
    const bool act = (ee < a.E) && (a.offsets[ee + 1] > a.offsets[ee]);
    uint64_t bal = __ballot(act);
    while (bal) {
      const int e = base + __ffsll((long long)bal) - 1;
      bal &= bal - 1;
      if ((seen++ % kG2Waves) != wv) continue;

      const int seg0 = a.offsets[e], seg1 = a.offsets[e + 1];
      const int me = segment_count(a.sorted_ids, seg0, seg1, a.P);
      const char* wr = reinterpret_cast<const char*>(a.w2) +
                       (((size_t)e * K + n0 + r16) * N + (size_t)g * Family<WT>::kPerLane) * WB;
      float scale = 1.0f;
      if (WT == DT_E4M3) scale = (*a.sh) * a.w2_scale[e];

      for (int c0 = 0; c0 < me; c0 += 16 * NCB) {
        const int ncb = min(NCB, (me - c0 + 15) / 16);
        const char* hr[NCB];
        bool hv[NCB];
        int tok[NCB];
        float rw[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          int col = c0 + cb * 16 + r16;
          bool ok = col < me;
          hv[cb] = ok;
          int pos = seg0 + (ok ? col : 0);
          int f = a.sorted_ids[pos];
          hr[cb] = hbase + (size_t)pos * N * HB;
          tok[cb] = ok ? f / a.topk : -1;
          rw[cb] = ok ? a.topk_w[f] : 0.0f;
        }
        f32x4 acc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0, 0, 0, 0};
        {
          G2Group<WT, NCB, U> A, B;
          int s = 0;
          g2_load(A, wr, hr, hv, s, nsteps, ncb);
          while (true) {
            if (s + U < nsteps) g2_load(B, wr, hr, hv, s + U, nsteps, ncb);
            g2_mma(A, s, nsteps, ncb, acc);
            s += U;
            if (s >= nsteps) break;
            if (s + U < nsteps) g2_load(A, wr, hr, hv, s + U, nsteps, ncb);
            g2_mma(B, s, nsteps, ncb, acc);
            s += U;
            if (s >= nsteps) break;
          }
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          if (cb < ncb && tok[cb] >= 0) {
            float* dst = my + (size_t)tok[cb] * 16 + 4 * g;
            const float m = scale * rw[cb];
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] += acc[cb][i] * m;
          }
        }
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < M * 4; i += blockDim.x) {
    const int t = i >> 2, q = (i & 3) * 4;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 0.0f;
      for (int w = 0; w < kG2Waves; ++w) s += acc_lds[((size_t)w * M + t) * 16 + q + j];
      v[j] = s;
    }
    store_out4<OT>(a.out, (size_t)t * K + n0 + q, v);
  }
}

template <>
__device__ __forceinline__ void store_out4<DT_F32>(void* out, size_t idx, const float v[4]) {
  st16(reinterpret_cast<float*>(out) + idx,
       i32x4{__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]),
             __float_as_int(v[3])});
}
template <>
__device__ __forceinline__ void store_out4<DT_BF16>(void* out, size_t idx, const float v[4]) {
  *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + idx) =
      make_uint2(pack_bf16x2(v[0], v[1]),
                 pack_bf16x2(v[2], v[3]));
}

// ================================================================== tile
//
// Workgroup = 4 waves over a block of BM token rows of one expert.  Each wave
// owns NA groups of 16 weight rows (loaded straight into registers); the
// token rows of the block are staged through LDS in chunks of 128 K values
// (KC steps), double-buffered, in the fragment order
// [step][lane group][row][32 bytes] so that a wave's 16 lanes of one group
// read 512 contiguous bytes.


template <int BT>
constexpr int tile_kc() {
  return 128 / fam_step<BT>();  // steps per 128-value chunk: bf16 2, E4M3 1
}

template <int BT, int BM>
struct TileLds {
  static constexpr int kChunkBytes = tile_kc<BT>() * 4 * BM * 32;
  static constexpr int kLoads = BM * tile_kc<BT>() * 8;  // 16-byte pieces per chunk
  static constexpr int kPerThread = (kLoads + 255) / 256;
};

template <int BT, int BM>
__device__ __forceinline__ void tile_fetch(const char* const rows[TileLds<BT, BM>::kPerThread],
                                           int chunk, i32x4 v[TileLds<BT, BM>::kPerThread]) {
  constexpr int KC = tile_kc<BT>();
#pragma unroll
  for (int j = 0; j < TileLds<BT, BM>::kPerThread; ++j) {
    const int idx = threadIdx.x + 256 * j;
    if (idx < TileLds<BT, BM>::kLoads) {
      const int c16 = idx % (KC * 8);
      v[j] = ld16(rows[j] + (size_t)chunk * KC * 128 + c16 * 16);
    }
  }
}

template <int BT, int BM>
__device__ __forceinline__ void tile_stash(char* lds, const i32x4 v[TileLds<BT, BM>::kPerThread]) {
  constexpr int KC = tile_kc<BT>();
#pragma unroll
  for (int j = 0; j < TileLds<BT, BM>::kPerThread; ++j) {
    const int idx = threadIdx.x + 256 * j;
    if (idx < TileLds<BT, BM>::kLoads) {
      const int r = idx / (KC * 8), c16 = idx % (KC * 8);
      const int st = c16 >> 3, grp = (c16 & 7) >> 1, half = c16 & 1;
      st16(lds + ((st * 4 + grp) * BM + r) * 32 + half * 16, v[j]);
    }
  }
}

// Main loop: acc[na][cb] += W rows (wrow[na]) x token tile, over Kdim.
template <int WT, int BT, int BM, int NA>
__device__ __forceinline__ void tile_mainloop(const char* const wrow[NA],
                                              const char* const trow[TileLds<BT, BM>::kPerThread],
                                              int Kdim, char* lds, f32x4 acc[NA][BM / 16]) {
  constexpr int KC = tile_kc<BT>();
  constexpr int NCB = BM / 16;
  constexpr int SB_W = fam_step<WT>() * Family<WT>::kBytes;
  constexpr int CB = TileLds<BT, BM>::kChunkBytes;
  static_assert(fam_step<WT>() == fam_step<BT>(), "operand families must match");
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int nchunks = Kdim / 128;

  i32x4 pre[TileLds<BT, BM>::kPerThread];
  tile_fetch<BT, BM>(trow, 0, pre);
  tile_stash<BT, BM>(lds, pre);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    char* cur = lds + (c & 1) * CB;
    if (c + 1 < nchunks) tile_fetch<BT, BM>(trow, c + 1, pre);
    Raw<WT> rw[NA][KC];
#pragma unroll
    for (int na = 0; na < NA; ++na)
#pragma unroll
      for (int st = 0; st < KC; ++st)
        rw[na][st] = load_raw<WT>(wrow[na] + (size_t)(c * KC + st) * SB_W);
#pragma unroll
    for (int st = 0; st < KC; ++st) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        Raw<BT> rb = load_raw<BT>(cur + ((st * 4 + g) * BM + cb * 16 + r16) * 32);
        auto b = to_op<BT>(rb);
#pragma unroll
        for (int na = 0; na < NA; ++na) acc[na][cb] = mma(to_op<WT>(rw[na][st]), b, acc[na][cb]);
      }
    }
    if (c + 1 < nchunks) tile_stash<BT, BM>(lds + ((c + 1) & 1) * CB, pre);
    __syncthreads();
  }
}

// XCD-aware order: the hardware deals consecutive workgroup ids round-robin
// over the 8 XCDs; remap so that each XCD walks a contiguous range of
// (weight tile, token block) tasks, token block fastest, keeping the blocks
// that share a weight tile on one L2.
__device__ __forceinline__ void tile_task(int& nt, int& mb) {
  const int nblk = gridDim.y, ntiles = gridDim.x;
  const int total = nblk * ntiles;
  const int lin = blockIdx.y * ntiles + blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = lin % 8, k = lin / 8;
  // XCD x owns tasks [start(x), start(x) + per + (x < rem)).
  const int task = xcd * per + min(xcd, rem) + k;
  nt = task / nblk;
  mb = task % nblk;
}

template <int WT, int XT, int BM>
__global__ __launch_bounds__(256) void gemm1_tile_kernel(GemmArgs a) {
  constexpr int NCB = BM / 16;
  constexpr int PT = TileLds<XT, BM>::kPerThread;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int nt, mb;
  tile_task(nt, mb);
  if (mb * BM >= *a.num_padded) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int e = a.block_expert[(mb * BM) / a.block_m];
  const int K = a.K, N = a.N;
  const int n0 = nt * 64 + wv * 16;
  constexpr int WB = Family<WT>::kBytes, XB = Family<XT>::kBytes;

  const char* w13 = reinterpret_cast<const char*>(a.w13);
  const char* wrow[2];
  wrow[0] = w13 + (((size_t)e * 2 * N + n0 + r16) * K + (size_t)g * Family<WT>::kPerLane) * WB;
  wrow[1] = wrow[0] + (size_t)N * K * WB;

  constexpr int KC = tile_kc<XT>();
  const char* trow[PT];
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const int idx = threadIdx.x + 256 * j;
    const int r = (idx < TileLds<XT, BM>::kLoads) ? idx / (KC * 8) : 0;
    int f = a.sorted_ids[mb * BM + r];
    if (f >= a.P) f = 0;
    trow[j] = reinterpret_cast<const char*>(a.x) + (size_t)(f / a.topk) * K * XB;
  }

  f32x4 acc[2][NCB];
#pragma unroll
  for (int na = 0; na < 2; ++na)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[na][cb] = f32x4{0, 0, 0, 0};
  tile_mainloop<WT, XT, BM, 2>(wrow, trow, K, lds, acc);

  float scale = 1.0f;
  if (WT == DT_E4M3) scale = (*a.sx) * a.w13_scale[e];
  float hmax = 0.0f;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int pos = mb * BM + cb * 16 + r16;
    if (a.sorted_ids[pos] < a.P) {
      float h[4], g4[4], u4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g4[i] = acc[0][cb][i] * scale;
        u4[i] = acc[1][cb][i] * scale;
        h[i] = silu(g4[i]) * u4[i];
      }
      const size_t idx = (size_t)pos * N + n0 + 4 * g;
      if (a.probe) {
        probe_store(a, (size_t)pos, n0 + 4 * g, g4, u4);
      } else if (WT == DT_E4M3) {
        st16(reinterpret_cast<float*>(a.h) + idx,
             i32x4{__float_as_int(h[0]), __float_as_int(h[1]), __float_as_int(h[2]),
                   __float_as_int(h[3])});
#pragma unroll
        for (int i = 0; i < 4; ++i) hmax = fmaxf(hmax, __builtin_fabsf(h[i]));
      } else {
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.h) + idx) =
            make_uint2(pack_bf16x2(h[0], h[1]),
                       pack_bf16x2(h[2], h[3]));
      }
    }
  }
  if (WT == DT_E4M3) {
    hmax = wave_max(hmax);
    if (lane == 0 && hmax > 0.0f) atomicMax(a.hmax_bits, __float_as_uint(hmax));
  }
}

// Down projection of one token block: y[pos] = scale * (W2 h); the routing
// weight is applied by the combine.
template <int WT, int BM>
__global__ __launch_bounds__(256) void gemm2_tile_kernel(GemmArgs a) {
  constexpr int HT = (WT == DT_E4M3) ? DT_E4M3 : DT_BF16;
  constexpr int NCB = BM / 16;
  constexpr int PT = TileLds<HT, BM>::kPerThread;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int nt, mb;
  tile_task(nt, mb);
  if (mb * BM >= *a.num_padded) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int e = a.block_expert[(mb * BM) / a.block_m];
  const int K = a.K, N = a.N;
  const int n0 = nt * 128 + wv * 32;
  constexpr int WB = Family<WT>::kBytes, HB = Family<HT>::kBytes;

  const char* w2 = reinterpret_cast<const char*>(a.w2);
  const char* wrow[2];
  wrow[0] = w2 + (((size_t)e * K + n0 + r16) * N + (size_t)g * Family<WT>::kPerLane) * WB;
  wrow[1] = wrow[0] + (size_t)16 * N * WB;

  constexpr int KC = tile_kc<HT>();
  const char* trow[PT];
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const int idx = threadIdx.x + 256 * j;
    const int r = (idx < TileLds<HT, BM>::kLoads) ? idx / (KC * 8) : 0;
    trow[j] = reinterpret_cast<const char*>(a.hq) + (size_t)(mb * BM + r) * N * HB;
  }

  f32x4 acc[2][NCB];
#pragma unroll
  for (int na = 0; na < 2; ++na)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[na][cb] = f32x4{0, 0, 0, 0};
  tile_mainloop<WT, HT, BM, 2>(wrow, trow, N, lds, acc);

  float scale = 1.0f;
  if (WT == DT_E4M3) scale = (*a.sh) * a.w2_scale[e];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int pos = mb * BM + cb * 16 + r16;
    if (a.sorted_ids[pos] < a.P) {
#pragma unroll
      for (int na = 0; na < 2; ++na) {
        const size_t idx = (size_t)pos * K + n0 + na * 16 + 4 * g;
        const float v[4] = {acc[na][cb][0] * scale, acc[na][cb][1] * scale, acc[na][cb][2] * scale,
                            acc[na][cb][3] * scale};
        if (a.ot == DT_BF16)
          store_out4<DT_BF16>(a.y, idx, v);
        else
          store_out4<DT_F32>(a.y, idx, v);
      }
    }
  }
}

// out[t] = sum over slots j (in routing order) of w[t, j] * y[pair_pos[t*k + j]]
// (y in the output's type: bf16 or fp32; the sum in fp32).  Workgroup = one
// token row (blockIdx.x) x kCombineCols columns (blockIdx.y); a thread takes
// CG groups of 8 columns, 2048 apart (bf16: two, so that a 4096-wide row
// fetches its slot positions and weights once and keeps 16 row loads in
// flight per thread); the slot positions and weights are wave-uniform.
template <int OT>
constexpr int combine_groups() { return OT == DT_BF16 ? 2 : 1; }

template <int OT>
__global__ __launch_bounds__(256) void combine_kernel(GemmArgs a) {
  constexpr int CG = combine_groups<OT>();
  constexpr int Q = (OT == DT_BF16) ? 1 : 2;  // 16-byte loads per 8-column group
  const int K = a.K;
  const int t = blockIdx.x;
  const int nb = blockIdx.y * 2048 * CG + threadIdx.x * 8;  // group c at nb + 2048 c
  float v[CG][8];
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) v[c][i] = 0.0f;
  // eight slots at a time: their rows are all requested before the first is
  // added, then added in slot order
  for (int j0 = 0; j0 < a.topk; j0 += 8) {
    int pos[8];
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = j0 + j < a.topk;
      pos[j] = ok ? a.pair_pos[(size_t)t * a.topk + j0 + j] : -1;
      w[j] = ok ? a.topk_w[(size_t)t * a.topk + j0 + j] : 0.0f;
    }
    i32x4 q[8][CG][Q];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        const int n = nb + 2048 * c;
        const size_t at = (size_t)(pos[j] < 0 ? 0 : pos[j]) * K + n;
#pragma unroll
        for (int u = 0; u < Q; ++u) {
          q[j][c][u] = i32x4{0, 0, 0, 0};
          if (pos[j] >= 0 && n < K)  // y is read exactly once: non-temporal
            q[j][c][u] = __builtin_nontemporal_load(
                (OT == DT_BF16) ? reinterpret_cast<const i32x4*>(reinterpret_cast<const uint16_t*>(a.y) + at)
                                : reinterpret_cast<const i32x4*>(reinterpret_cast<const float*>(a.y) + at + 4 * u));
        }
      }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (pos[j] < 0) continue;
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        if (OT == DT_BF16) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[c][2 * i] += w[j] * bf16_bits_to_f32((uint32_t)q[j][c][0][i] & 0xffffu);
            v[c][2 * i + 1] += w[j] * bf16_bits_to_f32((uint32_t)q[j][c][0][i] >> 16);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[c][i] += w[j] * __int_as_float(q[j][c][0][i]);
            v[c][4 + i] += w[j] * __int_as_float(q[j][c][Q - 1][i]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const int n = nb + 2048 * c;
    if (n < K) {
      const size_t o = (size_t)t * K + n;
      store_out4<OT>(a.out, o, v[c]);
      store_out4<OT>(a.out, o + 4, v[c] + 4);
    }
  }
}

__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ src,
                                                        uint16_t* __restrict__ dst, size_t n) {
  for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8; i < n;
       i += (size_t)gridDim.x * 256 * 8) {
    i32x4 p = pack_bf16x8(ld16(src + i), ld16(src + i + 4));
    st16(dst + i, p);
  }
}

// ------------------------------------------------------------------ launch

int device_cu_count() {
  // the first caller on a device queries it; a concurrent first call stores
  // the same value
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int c = cus[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
    c = n;
  }
  return c;
}

template <int WT, int XT>
static int g1s_dispatch(const GemmArgs& a, hipStream_t st, dim3 grid) {
  const int ncb = min((min(a.M, kStreamMaxM) + 15) / 16, kStreamMaxNcb);
  if (ncb <= 1)
    hipLaunchKernelGGL((gemm1_stream_kernel<WT, XT, 1>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm1_stream_kernel<WT, XT, kStreamMaxNcb>), grid, dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

int launch_gemm1_stream(const GemmArgs& a, hipStream_t st) {
  if (gemm1_ring_applies(a)) return launch_gemm1_ring(a, st);
  dim3 grid(a.N / 16, min(a.E, a.P));
  if (a.wt == DT_E4M3) return g1s_dispatch<DT_E4M3, DT_E4M3>(a, st, grid);
  if (a.wt == DT_BF16)
    return a.xt == DT_BF16 ? g1s_dispatch<DT_BF16, DT_BF16>(a, st, grid)
                           : g1s_dispatch<DT_BF16, DT_F32>(a, st, grid);
  return a.xt == DT_BF16 ? g1s_dispatch<DT_F32, DT_BF16>(a, st, grid)
                         : g1s_dispatch<DT_F32, DT_F32>(a, st, grid);
}

template <int WT, int OT>
static int g2s_dispatch(const GemmArgs& a, hipStream_t st) {
  const int ncb = min((min(a.M, kStreamMaxM) + 15) / 16, kStreamMaxNcb);
  dim3 grid(a.K / 16);
  size_t lds = (size_t)kG2Waves * a.M * 16 * sizeof(float);
  if (ncb <= 1)
    hipLaunchKernelGGL((gemm2_stream_kernel<WT, OT, 1>), grid, dim3(512), lds, st, a);
  else
    hipLaunchKernelGGL((gemm2_stream_kernel<WT, OT, kStreamMaxNcb>), grid, dim3(512), lds, st, a);
  return (int)hipGetLastError();
}

int launch_gemm2_stream(const GemmArgs& a, hipStream_t st) {
  if (a.wt == DT_E4M3)
    return a.ot == DT_BF16 ? g2s_dispatch<DT_E4M3, DT_BF16>(a, st) : g2s_dispatch<DT_E4M3, DT_F32>(a, st);
  if (a.wt == DT_BF16)
    return a.ot == DT_BF16 ? g2s_dispatch<DT_BF16, DT_BF16>(a, st) : g2s_dispatch<DT_BF16, DT_F32>(a, st);
  return a.ot == DT_BF16 ? g2s_dispatch<DT_F32, DT_BF16>(a, st) : g2s_dispatch<DT_F32, DT_F32>(a, st);
}

// Token block of the tile kernels: block_m, capped at 128 (a 256-row
// alignment block is processed as two halves of the same expert).
static inline int tile_bm(int block_m) { return block_m < 128 ? block_m : 128; }

template <int WT, int XT>
static int g1t_dispatch(const GemmArgs& a, hipStream_t st) {
  const int bm = tile_bm(a.block_m);
  dim3 grid(a.N / 64, a.max_blocks);
#define G1T(BM)                                                                         \
  if (bm == BM) {                                                                       \
    size_t lds = 2 * (size_t)TileLds<XT, BM>::kChunkBytes;                              \
    hipLaunchKernelGGL((gemm1_tile_kernel<WT, XT, BM>), grid, dim3(256), lds, st, a);  \
    return (int)hipGetLastError();                                                      \
  }
  G1T(16) G1T(32) G1T(64) G1T(128)
#undef G1T
  return -1;
}

int launch_gemm1_tile(const GemmArgs& a, hipStream_t st) {
  if (pfq_applies(a, true)) return launch_gemm1_pfq(a, st);
  if (pf_applies(a, true)) return launch_gemm1_prefill(a, st);
  // tile operands: bf16 family needs bf16 activations (f32 ones are cast first)
  if (a.wt == DT_E4M3) return g1t_dispatch<DT_E4M3, DT_E4M3>(a, st);
  if (a.wt == DT_BF16) return g1t_dispatch<DT_BF16, DT_BF16>(a, st);
  return g1t_dispatch<DT_F32, DT_BF16>(a, st);
}

template <int WT>
static int g2t_dispatch(const GemmArgs& a, hipStream_t st) {
  constexpr int HT = (WT == DT_E4M3) ? DT_E4M3 : DT_BF16;
  const int bm = tile_bm(a.block_m);
  dim3 grid(a.K / 128, a.max_blocks);
#define G2T(BM)                                                                   \
  if (bm == BM) {                                                                 \
    size_t lds = 2 * (size_t)TileLds<HT, BM>::kChunkBytes;                        \
    hipLaunchKernelGGL((gemm2_tile_kernel<WT, BM>), grid, dim3(256), lds, st, a); \
    return (int)hipGetLastError();                                                \
  }
  G2T(16) G2T(32) G2T(64) G2T(128)
#undef G2T
  return -1;
}

int launch_gemm2_tile(const GemmArgs& a, hipStream_t st) {
  if (pfq_applies(a, false)) return launch_gemm2_pfq(a, st);
  if (pf_applies(a, false)) return launch_gemm2_prefill(a, st);
  if (a.wt == DT_E4M3) return g2t_dispatch<DT_E4M3>(a, st);
  if (a.wt == DT_BF16) return g2t_dispatch<DT_BF16>(a, st);
  return g2t_dispatch<DT_F32>(a, st);
}

int launch_combine(const GemmArgs& a, hipStream_t st) {
  if (a.ot == DT_BF16) {
    const int cols = 2048 * combine_groups<DT_BF16>();
    hipLaunchKernelGGL(combine_kernel<DT_BF16>, dim3((unsigned)a.M, (unsigned)((a.K + cols - 1) / cols)),
                       dim3(256), 0, st, a);
  } else {
    const int cols = 2048 * combine_groups<DT_F32>();
    hipLaunchKernelGGL(combine_kernel<DT_F32>, dim3((unsigned)a.M, (unsigned)((a.K + cols - 1) / cols)),
                       dim3(256), 0, st, a);
  }
  return (int)hipGetLastError();
}

int launch_cast_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t st) {
  size_t want = (n + 2047) / 2048;
  int g = (int)(want < 4096 ? (want ? want : 1) : 4096);
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(g), dim3(256), 0, st, src, dst, n);
  return (int)hipGetLastError();
}

}  // namespace moe
