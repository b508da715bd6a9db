// ring.hpp -- the LDS weight ring of the decode expert GEMMs, shared by the
// stand-alone ring kernels (ring.hip) and the single-launch decode forward
// (fused.hip).
//
// Both expert GEMMs of the decode path stream the expert
// weights through an LDS ring filled by direct-to-LDS loads (gfx950
// global_load_lds_dwordx4).
//
// The expert product is A[M,K] x B[K,N] with few token rows M at decode
// ("Amazon SageMaker AI 上的 Mixture-of-Experts 内核工程优化", section "Swap-AB
// for WGMMA utilization"); the weights are the bytes to move, each active
// expert's rows exactly once ("... section "Backend routing for FP8 tensor
// quantization": data read from HBM once and kept on chip).
//
// Why a ring: an MFMA row operand needs 16 different weight rows per wave
// instruction, and reading them straight into registers makes every load
// touch 16 rows x 64 bytes, which sustains about 5.4 TB/s on MI355X.  Here
// each direct-to-LDS wave instruction reads 2 rows x 512 contiguous bytes
// (about 6 TB/s in the same test), the LDS holds kRingD stages, and the MFMA
// fragments are read back from LDS.  The second row of each DMA block has its
// 128-byte halves swapped (the source addresses are permuted, the LDS writes
// stay lane-ordered), which puts the 16 rows one ds_read_b128 touches on 16
// different bank groups.
//
// Stage: 512 bytes of each of 32 rows (gate/up: 16 gate + 16 up rows of one
// expert; down: 32 consecutive rows of w2), 4 K-steps, one step per wave of
// the 4 streaming waves.  Each wave keeps its own operand fragments (x rows
// for gate/up, h rows for down) of the kRingD - 1 stages in flight in
// registers, issued together with the stage's DMA so that a single in-order
// vmcnt wait covers both.
#pragma once

#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace moe {

constexpr int kRingD = 4;               // stages in the ring
constexpr int kRingRowBytes = 512;      // bytes of one weight row per stage
constexpr int kPairStride = 2 * kRingRowBytes + 16;  // LDS bytes of a 2-row DMA block
constexpr int kG1RingRows = 32;         // 16 gate + 16 up rows
constexpr int kG1StageBytes = (kG1RingRows / 2) * kPairStride;
constexpr int kRingAux = 2;             // cache-policy bits of the weight DMA (2: nt)

__device__ __forceinline__ int ring_off(int r, int b) {
  return (r >> 1) * kPairStride + (r & 1) * kRingRowBytes + (b ^ ((r & 1) << 7));
}

// s_waitcnt vmcnt(N) through the builtin, so that the compiler's own wait
// insertion knows these loads have landed (an inline-asm wait is opaque to
// it).  GFX9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4]
// at [15:14]; expcnt and lgkmcnt left at their maxima (no wait).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
// Keeps one ring stage's loads (register x/h fragments and LDS DMA) in
// program order relative to the next stage's.  The hand-counted vmcnt waits
// assume every stage's instructions were issued before any of a later
// stage's; without a fence the scheduler may hoist a later stage's DMA above
// an earlier stage's register loads (which wait for the token ids), and a
// wait for "all but the last (D-1) stages" then leaves part of the stage
// being read still in flight.
__device__ __forceinline__ void stage_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Workgroup barrier without the fence of __syncthreads (which would also wait
// for the ring's outstanding loads); the empty asm keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------ expert rings
//
// Both expert GEMMs of the decode path: one launch of a fixed number of
// workgroups (WPC per CU) that walk a static list of tasks without draining
// the ring between them.  Task = (column group, 32-row block): a column group
// is 16*NCB consecutive sorted positions -- part of one alignment block when
// block_m is a multiple of 16*NCB, else two consecutive 16-row blocks of one
// expert (pair_heads) -- and the row block is
// 32 weight rows of the block's expert -- for gate/up (G1) gate rows
// n0..n0+15 with the matching up rows, for the down projection 32
// consecutive rows of w2.  Tasks are numbered group-major; workgroup w takes
// tasks w, w + G, w + 2G, ... (G workgroups), so every workgroup streams the
// same number of weight bytes (to one task), the ring fills and drains once
// per workgroup instead of once per row block, and at any moment the
// workgroups read neighbouring tasks (the order a one-task-per-workgroup
// launch would dispatch them in).  Everything a task needs before its first
// load -- expert, dequant scale, row block, the operand row of each column --
// is read into an LDS table row when the workgroup starts, so that switching
// tasks inside the stream reads only LDS and never waits on the
// vector-memory counter the ring runs on.
//
// At the end of a task the four K-slices are summed by a fifth wave from
// partial sums the streaming waves leave in a small LDS area beside the
// ring, while they already work on the next task's stages.  Gate/up writes
// SiLU(gate) * up to h; the down projection writes each pair's 32 output
// features, dequantised but not yet weighted, to y, and the combine kernel
// sums the top-k rows of every token with their routing weights.

constexpr int kPRedBytesPerCb = 4 * 2 * 4 * kWave * 4;  // 4 streaming waves x 2 halves x 4 regs x lanes

template <int WT, int NCB, int D, bool G1>
struct PRing {
  static constexpr int SB = 128;          // bytes per K-step of a row
  static constexpr int NI = 4 + 2 * NCB;  // vector-memory instructions per issue
  static constexpr int WB = Family<WT>::kBytes;
  static constexpr int CPG = 16 * NCB;    // columns per group
  // table row: expert, scale bits, row block, first sorted position, K stage
  // the task starts at, then one byte per column: 255 for padding, else for
  // gate/up the token row of x (the decode path has at most 64 tokens); the
  // down projection reads h at the column's sorted position
  static constexpr int TW = 5 + CPG / 4;
  static constexpr int kPad = 255;
  char* ring;
  const int* tab;
  const char* w;   // expert weights [E][rows][kdim]
  const char* xb;  // operand rows + this lane's 32-byte offset within a K-step
  size_t wrow;     // bytes of one weight row = bytes of one operand row
  int wrows;       // weight rows per expert
  int half;        // G1: row offset of the up half (N)
  int ns, wv, r16, lrow, lb, ng;
  // issue cursor: table row (task of this workgroup), stage within the task
  int iq, ik;
  int irot;  // K stage the task starts at (tasks walk K from different offsets)
  const char* src[4];
  const char* xr[NCB];
  int dst[4];
  Raw<WT> xs[D][NCB];

  __device__ __forceinline__ void set_task(int q) {
    const int* row = tab + q * TW;
    const int e = row[0], rb = row[2];
    irot = row[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = 2 * (4 * wv + qq) + lrow;
      int grow;
      if constexpr (G1)
        grow = (r < 16) ? (16 * rb + r) : (half + 16 * rb + r - 16);
      else
        grow = 32 * rb + r;
      src[qq] = w + ((size_t)e * wrows + grow) * wrow + lb;
    }
    const uint8_t* col8 = reinterpret_cast<const uint8_t*>(row + 5);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = cb * 16 + r16;
      int xrow;
      if constexpr (G1) {
        xrow = col8[c] == kPad ? 0 : col8[c];
      } else {
        // padding columns read the group's first row (always inside h); their
        // sums are dropped
        xrow = col8[c] == kPad ? row[3] : row[3] + c;
      }
      xr[cb] = xb + (size_t)xrow * wrow;
    }
  }

  template <int SLOT>
  __device__ __forceinline__ void issue() {
    const int kc = ik + irot < ns ? ik + irot : ik + irot - ns;  // K stage loaded now
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      xs[SLOT][cb] = load_raw<WT>(xr[cb] + (size_t)(kc * 4 + wv) * SB);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(src[qq] + (size_t)kc * kRingRowBytes),
          reinterpret_cast<void*>(ring + SLOT * kG1StageBytes + dst[qq]), 16, 0, kRingAux);
    stage_fence();
    if (++ik == ns) {
      ik = 0;
      if (++iq < ng) set_task(iq);
    }
  }

  // One stage: refill (ISSUE) or drain, then this wave's K-step of the slot.
  template <int SLOT, bool ISSUE>
  __device__ __forceinline__ void body(f32x4 acc0[NCB], f32x4 acc1[NCB], int g) {
    if constexpr (ISSUE) {
      issue<(SLOT + D - 1) % D>();
      wait_vmcnt<(D - 1) * NI>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();
    const char* sb = ring + SLOT * kG1StageBytes;
    const int b = wv * SB + g * 32;
    Raw<WT> a0, a1;
    const int o0 = ring_off(r16, b), o1 = ring_off(16 + r16, b);
    a0.q[0] = ld16(sb + o0);
    a0.q[1] = ld16(sb + o0 + 16);
    a1.q[0] = ld16(sb + o1);
    a1.q[1] = ld16(sb + o1 + 16);
    const auto A0 = to_op<WT>(a0);
    const auto A1 = to_op<WT>(a1);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const auto X = to_op<WT>(xs[SLOT][cb]);
      acc0[cb] = mma(A0, X, acc0[cb]);
      acc1[cb] = mma(A1, X, acc1[cb]);
    }
  }
};

constexpr int kRingWaves = 4;
constexpr int kRingThreads = (kRingWaves + 1) * kWave;
constexpr int kPairMaxE = 4 * kRingThreads;  // experts the pairing scan covers (4 per thread)

// Alignment blocks of 16 rows and experts with more tokens than one block
// holds: a 16-column task streams the expert's weight rows once per block.
// Column groups of two consecutive blocks of one expert (counted from the
// expert's first block; expert_offsets holds the padded segment starts) read
// them once per two blocks, at the price of 32-column tasks everywhere (the
// second block of a group may belong to the next expert, and its columns are
// then padding).  pair_scan counts the groups, ceil(blocks / 2) per expert,
// and gives this thread's first group index; pair_heads then writes the
// first block of every group in group order.  wsum: kRingThreads / kWave ints
// of LDS.  Every thread of the workgroup calls both (they synchronise it).
__device__ __forceinline__ int pair_scan(const GemmArgs& a, int* wsum, int& my_base) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (a.E + kRingThreads - 1) / kRingThreads;  // <= 4 (host check)
  const int e0 = min(tid * per, a.E), e1 = min(e0 + per, a.E);
  int c = 0;
  for (int e = e0; e < e1; ++e) c += ((a.offsets[e + 1] - a.offsets[e]) / a.block_m + 1) >> 1;
  int v = c;  // inclusive scan over the wave
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  if (lane == kWave - 1) wsum[wv] = v;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kRingThreads / kWave; ++i) {
    const int t = wsum[i];
    base += i < wv ? t : 0;
    total += t;
  }
  my_base = base + v - c;
  __syncthreads();  // wsum is read before anything reuses the space
  return total;
}

__device__ __forceinline__ void pair_heads(const GemmArgs& a, int my_base, int* heads) {
  const int tid = threadIdx.x;
  const int per = (a.E + kRingThreads - 1) / kRingThreads;
  const int e0 = min(tid * per, a.E), e1 = min(e0 + per, a.E);
  int k = my_base;
  for (int e = e0; e < e1; ++e) {
    const int first = a.offsets[e] / a.block_m, nblk = (a.offsets[e + 1] - a.offsets[e]) / a.block_m;
    for (int j = 0; j < nblk; j += 2) heads[k++] = first + j;
  }
  __syncthreads();
}

// ------------------------------------------------- single-launch hooks
//
// Inside one launch, data that a workgroup hands to workgroups on other XCDs
// (each XCD has its own L2) is written with device-scope stores (sc1: the
// store completes at the device-coherent level) and read with device-scope
// loads where the reader's L2 may already hold the line.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kCohAux = 16;  // sc1
__device__ __forceinline__ void coh_st16(__amdgpu_buffer_rsrc_t r, uint32_t off, i32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)off, 0, kCohAux);
}
__device__ __forceinline__ void coh_st8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{v.x, v.y}, r, (int)off, 0, kCohAux);
}
__device__ __forceinline__ i32x4 coh_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCohAux));
}

// What the single-launch forward (fused.hip) changes in ring_run: the scale
// of the activation operand comes in as a value (it was reduced over the
// grid inside the launch), the gate/up epilogue leaves its max |h| in LDS
// instead of raising a global maximum, and h and y are stored
// device-coherent in tiled layouts that give every 128-byte line one writer
// (h [N / 16][rows][16], y [K / 32][rows][32], rows = the padded pair
// count).
struct RingFused {
  float act_scale;  // s_x (gate/up) or s_h (down)
  float* hmax;      // LDS slot of the gate/up epilogue wave's max |h|
};

// Workgroup = kRingWaves streaming waves (each one K-step of every stage) and
// one epilogue wave.  The epilogue wave sums the streaming waves' partial
// sums at the end of every task and does all the global stores, while the
// streaming waves already load and multiply the next task's stages: their
// loop then holds only loads, so the compiler can keep counting the loads
// in flight (a store among them makes it wait for every outstanding load
// before the next MFMA, which empties the ring).

// heads == nullptr: column groups are blocks or parts of blocks (block_m a
// multiple of 16 * NCB); else the ngrp groups of two 16-row blocks that
// pair_heads listed.  FUSED: the single-launch variant (RingFused).
template <int WT, int NCB, int D, bool G1, bool FUSED = false>
__device__ __forceinline__ void ring_run(const GemmArgs& a, int GT, char* lds, const int* heads, int ngrp,
                                         RingFused fz = RingFused{}) {
  using R_t = PRing<WT, NCB, D, G1>;
  constexpr int CPG = R_t::CPG, TW = R_t::TW, WB = R_t::WB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int bm = a.block_m;
  // gate/up: [E][2N][K] weights, out rows N per half, K-dim K; down: [E][K][N]
  // weights, 32 of its K rows per task, K-dim N
  const int kdim = G1 ? a.K : a.N;
  const int ns = kdim * WB / kRingRowBytes;
  const int nrb = G1 ? a.N / 16 : a.K / 32;
  const int npb = bm > CPG ? bm / CPG : 1;  // column groups per alignment block
  const int nb = *a.num_padded / bm;
  const bool span = heads != nullptr;  // groups of two blocks
  if (!span) ngrp = nb * npb;

  f32x4* red = reinterpret_cast<f32x4*>(lds + D * kG1StageBytes);
  int* tab = reinterpret_cast<int*>(lds + D * kG1StageBytes + NCB * kPRedBytesPerCb);
  const long long ntask = (long long)ngrp * nrb;
  const long long G = gridDim.x, w = blockIdx.x;
  const long long ntw = w < ntask ? (ntask - 1 - w) / G + 1 : 0;  // tasks w, w + G, ...
  if (ntw <= 0) return;  // uniform over the workgroup
  // never clamped: the host sizes GT for the longest task list
  const int ng = ntw < GT ? (int)ntw : GT;
  // partial sums as [wave][half][cb][lane] x 4 floats: one 16-byte LDS access
  // per accumulator
  auto part = [&](int w2, int h2, int cb) { return red + ((w2 * 2 + h2) * NCB + cb) * kWave + lane; };

  // ---- task table: each task's expert, dequant scale, row block, first
  // sorted position and first K stage, then its column bytes.  The
  // first K stage is a hash of the task index: workgroups that start
  // together would otherwise all read the same 512-byte column of their rows
  // at the same time (measured on E4M3 gate/up weights at 32 and 64 tokens:
  // 8-9% slower when every task starts at stage 0).
  // A group's columns are the sorted positions pos0 .. pos0 + CPG - 1 with
  // pos0 = (first block) * bm + (part of the block) * CPG; a spanning group's
  // columns in a block of another expert, or past the last block, are padding.
  for (int i = tid; i < ng * CPG; i += kRingThreads) {
    const int q = i / CPG, col = i - q * CPG;
    const long long t = w + q * G;
    const int gq = (int)(t / nrb);
    int b = R_t::kPad;
    if (span) {
      const int blk = heads[gq], bb = blk + col / bm;
      if (bb < nb && a.block_expert[bb] == a.block_expert[blk]) {
        const int f = a.sorted_ids[blk * bm + col];
        if (f < a.P) b = G1 ? f / a.topk : 0;
      }
    } else {
      const int blk = gq / npb, lc = (gq - blk * npb) * CPG + col;
      if (lc < bm) {
        const int f = a.sorted_ids[blk * bm + lc];
        if (f < a.P) b = G1 ? f / a.topk : 0;
      }
    }
    reinterpret_cast<uint8_t*>(tab + q * TW + 5)[col] = (uint8_t)b;
  }
  for (int q = tid; q < ng; q += kRingThreads) {
    const long long t = w + q * G;
    const int gq = (int)(t / nrb);
    const int blk = span ? heads[gq] : gq / npb;
    const int e = a.block_expert[blk];
    float sc = 1.0f;
    if (WT == DT_E4M3) {
      const float as = FUSED ? fz.act_scale : (G1 ? *a.sx : *a.sh);
      sc = as * (G1 ? a.w13_scale[e] : a.w2_scale[e]);
    }
    tab[q * TW] = e;
    tab[q * TW + 1] = __float_as_int(sc);
    tab[q * TW + 2] = (int)(t - (long long)gq * nrb);
    tab[q * TW + 3] = blk * bm + (span ? 0 : (gq - blk * npb) * CPG);
    tab[q * TW + 4] = (int)((((unsigned)t * 2654435761u) >> 16) % (unsigned)ns);
  }
  __syncthreads();

  const int total = ng * ns;  // stages of this workgroup

  if (wv == kRingWaves) {
    // ---- epilogue wave: the same two barriers per stage as the streaming
    // waves; after the second barrier of a task's last stage the partial
    // sums are complete, and they stay untouched until the streaming waves
    // pass the next stage's first barrier, which waits for this wave
    float hmax = 0.0f;
    int cq = 0, ck = 0;
    for (int p = 0; p < total; ++p) {
      wg_barrier();
      wg_barrier();
      if (++ck < ns) continue;
      ck = 0;
      const int* row = tab + cq * TW;
      const float scale = __int_as_float(row[1]);
      const int rb = row[2];
      const size_t pos0 = (size_t)row[3];
      const uint8_t* col8 = reinterpret_cast<const uint8_t*>(row + 5);
      ++cq;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f32x4 s0 = *part(0, 0, cb), s1 = *part(0, 1, cb);
#pragma unroll
        for (int w2 = 1; w2 < kRingWaves; ++w2) {
          const f32x4 p0 = *part(w2, 0, cb), p1 = *part(w2, 1, cb);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s0[i] += p0[i];
            s1[i] += p1[i];
          }
        }
        const int col = cb * 16 + r16;
        if (col8[col] == R_t::kPad) continue;
        float v0[4], v1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v0[i] = s0[i] * scale;
          v1[i] = s1[i] * scale;
        }
        const size_t pr = pos0 + col;
        if constexpr (G1) {
          const int N = a.N, n0 = 16 * rb;
          float h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = silu(v0[i]) * v1[i];
          if (a.probe) {
            probe_store(a, pr, n0 + 4 * g, v0, v1);
          } else if (WT == DT_E4M3) {
            const i32x4 hv{__float_as_int(h[0]), __float_as_int(h[1]), __float_as_int(h[2]),
                           __float_as_int(h[3])};
            if constexpr (FUSED)  // tiled [N / 16][rows][16]: one writer per 128-byte line
              coh_st16(dev_rsrc(a.h), (uint32_t)((((size_t)rb * nb * bm + pr) * 16 + 4 * g) * 4), hv);
            else
              st16(reinterpret_cast<float*>(a.h) + pr * N + n0 + 4 * g, hv);
#pragma unroll
            for (int i = 0; i < 4; ++i) hmax = fmaxf(hmax, __builtin_fabsf(h[i]));
          } else {
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.h) + pr * N + n0 + 4 * g) =
                make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
          }
        } else {
          const size_t o = pr * a.K + 32 * rb + 4 * g;  // rows 4g.. and 16 + 4g.. of the block
          // FUSED: tiled [K / 32][rows][32], one writer per 128-byte line
          const size_t ot = ((size_t)rb * nb * bm + pr) * 32 + 4 * g;
          if (FUSED && a.ot == DT_BF16) {
            const auto yr = dev_rsrc(a.y);
            coh_st8(yr, (uint32_t)(ot * 2), make_uint2(pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3])));
            coh_st8(yr, (uint32_t)((ot + 16) * 2),
                    make_uint2(pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])));
          } else if (FUSED) {
            const auto yr = dev_rsrc(a.y);
            coh_st16(yr, (uint32_t)(ot * 4),
                     i32x4{__float_as_int(v0[0]), __float_as_int(v0[1]), __float_as_int(v0[2]), __float_as_int(v0[3])});
            coh_st16(yr, (uint32_t)((ot + 16) * 4),
                     i32x4{__float_as_int(v1[0]), __float_as_int(v1[1]), __float_as_int(v1[2]), __float_as_int(v1[3])});
          } else if (a.ot == DT_BF16) {
            uint16_t* y = reinterpret_cast<uint16_t*>(a.y);
            *reinterpret_cast<uint2*>(y + o) =
                make_uint2(pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]));
            *reinterpret_cast<uint2*>(y + o + 16) =
                make_uint2(pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3]));
          } else {
            float* y = reinterpret_cast<float*>(a.y);
            st16(y + o, i32x4{__float_as_int(v0[0]), __float_as_int(v0[1]),
                              __float_as_int(v0[2]), __float_as_int(v0[3])});
            st16(y + o + 16, i32x4{__float_as_int(v1[0]), __float_as_int(v1[1]),
                                   __float_as_int(v1[2]), __float_as_int(v1[3])});
          }
        }
      }
    }
    if (G1 && WT == DT_E4M3) {
      hmax = wave_max(hmax);
      if constexpr (FUSED) {
        if (lane == 0) *fz.hmax = hmax;
      } else {
        if (lane == 0 && hmax > 0.0f) atomicMax(a.hmax_bits, __float_as_uint(hmax));
      }
    }
    return;
  }

  // ---- streaming waves
  R_t R;
  R.ring = lds;
  R.tab = tab;
  R.w = reinterpret_cast<const char*>(G1 ? a.w13 : a.w2);
  R.xb = reinterpret_cast<const char*>(G1 ? a.x : a.hq) + g * 32;
  R.wrow = (size_t)kdim * WB;
  R.wrows = G1 ? 2 * a.N : a.K;
  R.half = a.N;
  R.ns = ns;
  R.wv = wv;
  R.r16 = r16;
  R.lrow = lane >> 5;
  R.lb = ((lane & 31) << 4) ^ (R.lrow << 7);
  R.ng = ng;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) R.dst[qq] = (4 * wv + qq) * kPairStride;
  R.iq = 0;
  R.ik = 0;
  R.set_task(0);

  int ck = 0;  // stage within the task being multiplied
  f32x4 acc0[NCB], acc1[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc0[cb] = acc1[cb] = f32x4{0, 0, 0, 0};

  // Stage p uses slot p % D.  The steady loop holds only stages that refill
  // the ring (stage p + D - 1 exists) in whole trips of D, so every slot index
  // is static (the operand fragments live in registers) and every path
  // through the loop issues the same loads: the compiler can then tell which
  // fragments have landed from the explicit waits alone.  A branch between
  // refilling and draining stages inside the loop makes it wait for all
  // loads in flight before some MFMAs.
  auto stage = [&](auto slot, auto refill) __attribute__((always_inline)) {
    R.template body<decltype(slot)::value, decltype(refill)::value>(acc0, acc1, g);
    if (++ck == ns) {  // task done: hand the partial sums to the epilogue wave
      ck = 0;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        *part(wv, 0, cb) = acc0[cb];
        *part(wv, 1, cb) = acc1[cb];
        acc0[cb] = acc1[cb] = f32x4{0, 0, 0, 0};
      }
    }
    wg_barrier();
  };
  using Refill = std::true_type;
  using Drain = std::false_type;

  if (total < D - 1) {  // fewer stages than the ring holds: load all, then drain
    static_for<0, D - 1>([&](auto i) {
      if (decltype(i)::value < total) R.template issue<decltype(i)::value>();
    });
    static_for<0, D - 1>([&](auto i) {
      if (decltype(i)::value < total) stage(i, Drain{});
    });
    return;
  }
  static_for<0, D - 1>([&](auto i) { R.template issue<decltype(i)::value>(); });
  const int n_issue = total - (D - 1);  // stages that refill the ring
  int st = 0;
  for (; st + D <= n_issue; st += D) static_for<0, D>([&](auto i) { stage(i, Refill{}); });
  // the last n_issue % D refilling stages, then D - 1 draining ones
  const int rem = n_issue - st;  // 0 .. D - 1
  static_for<0, D>([&](auto rr) {
    constexpr int RR = decltype(rr)::value;
    if (rem == RR) {
      static_for<0, RR>([&](auto i) { stage(i, Refill{}); });
      static_for<0, D - 1>([&](auto j) {
        stage(std::integral_constant<int, (RR + decltype(j)::value) % D>{}, Drain{});
      });
    }
  });
}

// NCB = 0: 16-row alignment blocks, column groups of one or two blocks chosen
// here from expert_offsets -- two when that removes at least an eighth of the
// groups (the 32-column tasks cost about 2% where every expert fits one
// block: measured on 64-token E4M3 gate/up with uniform routing).  The
// two-block path runs a ring one stage shorter, so that both paths leave room
// for two workgroups per CU (four stages and the partial sums of 32 columns
// do not).
constexpr int kPairGain = 8;

// Host-side sizes of a ring launch of WPC workgroups per CU: the task table
// is sized for the longest task list a workgroup can get (capacity bound /
// G, rounded up, plus one).
template <int WT, int NCB, int D, int WPC, bool G1>
struct RingSize {
  using R_t = PRing<WT, NCB == 0 ? 2 : NCB, D, G1>;  // NCB = 0: table rows of the wider groups
  static int table_rows(const GemmArgs& a) {
    const int bm = a.block_m;
    const long long npb = bm > R_t::CPG ? bm / R_t::CPG : 1;
    const long long cap = (long long)a.P + (long long)min(a.E, a.P) * (bm - 1);
    const long long ntask = (cap + bm - 1) / bm * npb * (G1 ? a.N / 16 : a.K / 32);
    const long long G = (long long)WPC * device_cu_count();
    return (int)((ntask + G - 1) / G) + 1;
  }
  static size_t lds(const GemmArgs& a) {
    const size_t tab = (size_t)table_rows(a) * R_t::TW * sizeof(int);
    if (NCB == 0)  // the larger of the two paths' needs
      return max((size_t)D * kG1StageBytes + kPRedBytesPerCb + tab,
                 (size_t)(D - 1) * kG1StageBytes + 2 * kPRedBytesPerCb + tab);
    return (size_t)D * kG1StageBytes + NCB * kPRedBytesPerCb + tab;
  }
  static bool fits(const GemmArgs& a) { return lds(a) <= (size_t)160 * 1024 / WPC; }
};

// 16-row alignment blocks: NCB = 0 (one- or two-block column groups, chosen
// by the kernel) where the pairing scan covers E and the group heads fit in
// the ring's space.
inline bool ring_pair_fits(const GemmArgs& a) {
  const long long cap = (long long)a.P + (long long)min(a.E, a.P) * (a.block_m - 1);
  const long long nb = (cap + a.block_m - 1) / a.block_m;
  return a.E <= kPairMaxE && nb * 4 <= (long long)(kRingD - 1) * kG1StageBytes;
}

// Both rings need bf16 or E4M3 weights with an operand of the same type
// (gate/up: x; down: h, which the layer keeps in the weights' type) and
// K-dimension rows of whole 512-byte stages.
inline bool ring_rows(const GemmArgs& a, int kdim) {
  const long long row = (long long)kdim * (a.wt == DT_BF16 ? 2 : 1);
  return row % kRingRowBytes == 0;
}

}  // namespace moe
