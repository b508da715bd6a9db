// ring.hip -- decode gate/up GEMM that streams expert weights through an LDS
// ring filled by direct-to-LDS loads (gfx950 global_load_lds_dwordx4).
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
// Gate/up stage: 512 bytes of each of 32 rows (16 gate + 16 up rows of one
// expert, 4 K-steps), one step per wave of a 4-wave workgroup.  Each wave
// keeps its own x fragments of the kRingD - 1 stages in flight in registers,
// issued together with the stage's DMA so that a single in-order vmcnt wait
// covers both.
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
constexpr int kRingNcbMax = 2;

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

// ------------------------------------------------------------ gate/up ring
//
// One launch of a fixed number of workgroups (WPC per CU) that walk a static
// list of tasks without draining the ring between them.  Task = (column group, 16-row block): a column group
// is 16*NCB consecutive positions of one alignment block (block_m = 16*NCB, or
// a multiple of it, then one block is several groups), and a row block is
// gate rows n0..n0+15 with the matching up rows, of the block's expert.  Tasks
// are numbered group-major; workgroup w takes tasks w, w + G, w + 2G, ... (G
// workgroups), so every workgroup streams the same number of weight bytes (to
// one task), the ring fills and drains once per workgroup instead of once per
// row block, and at any moment the workgroups read neighbouring tasks (the
// order a one-task-per-workgroup launch would dispatch them in).  Everything a
// task needs before its first load -- expert, dequant scale, row block, the
// token row of each column -- is read into an LDS table row when the
// workgroup starts, so that switching tasks inside the stream reads only LDS
// and never waits on the vector-memory counter the ring runs on.
//
// At the end of a task the four K-slices are summed by wave 0 (waves 1..3
// leave their partial sums in a small LDS area beside the ring) while the
// other waves already work on the next task's stages.

constexpr int kPRedBytesPerCb = 3 * 2 * 4 * kWave * 4;  // waves 1..3 x gate/up x 4 regs x lanes

template <int WT, int NCB, int D>
struct PRing {
  static constexpr int SB = 128;          // bytes per K-step of a row
  static constexpr int NI = 4 + 2 * NCB;  // vector-memory instructions per issue
  static constexpr int WB = Family<WT>::kBytes;
  static constexpr int CPG = 16 * NCB;    // columns per group
  // table row: expert, scale bits, row block, first sorted position, K stage
  // the task starts at, then the token row of every column (-1: padding)
  static constexpr int TW = CPG + 5;
  char* ring;
  float* red;
  const int* tab;
  const char* w13;
  const char* xb;  // x + this lane's 32-byte offset within a K-step
  int K, N, ns, wv, r16, lrow, lb, ng;
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
    const int n0 = rb * 16;
    irot = row[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = 2 * (4 * wv + qq) + lrow;
      const int grow = (r < 16) ? (n0 + r) : (N + n0 + r - 16);
      src[qq] = w13 + ((size_t)e * 2 * N + grow) * K * WB + lb;
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int t = row[5 + cb * 16 + r16];
      xr[cb] = xb + (size_t)(t < 0 ? 0 : t) * K * WB;
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
  __device__ __forceinline__ void body(f32x4 accg[NCB], f32x4 accu[NCB], int g) {
    if constexpr (ISSUE) {
      issue<(SLOT + D - 1) % D>();
      wait_vmcnt<(D - 1) * NI>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();
    const char* sb = ring + SLOT * kG1StageBytes;
    const int b = wv * SB + g * 32;
    Raw<WT> ag, au;
    const int og = ring_off(r16, b), ou = ring_off(16 + r16, b);
    ag.q[0] = ld16(sb + og);
    ag.q[1] = ld16(sb + og + 16);
    au.q[0] = ld16(sb + ou);
    au.q[1] = ld16(sb + ou + 16);
    const auto A = to_op<WT>(ag);
    const auto U = to_op<WT>(au);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const auto X = to_op<WT>(xs[SLOT][cb]);
      accg[cb] = mma(A, X, accg[cb]);
      accu[cb] = mma(U, X, accu[cb]);
    }
  }
};

template <int WT, int NCB, int D, int WPC>
__global__ __launch_bounds__(256, WPC) void gemm1_ring_kernel(GemmArgs a, int GT) {
  using R_t = PRing<WT, NCB, D>;
  constexpr int CPG = R_t::CPG, TW = R_t::TW, WB = R_t::WB;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int K = a.K, N = a.N, bm = a.block_m;
  const int ns = K * WB / kRingRowBytes;
  const int nrb = N / 16;
  const int npb = bm > CPG ? bm / CPG : 1;  // column groups per alignment block
  const long long ntask = (long long)(*a.num_padded / bm) * npb * nrb;
  const long long G = gridDim.x, w = blockIdx.x;
  const long long ntw = w < ntask ? (ntask - 1 - w) / G + 1 : 0;  // tasks w, w + G, ...
  if (ntw <= 0) return;  // uniform over the workgroup
  // never clamped: the host sizes GT for the longest task list
  const int ng = ntw < GT ? (int)ntw : GT;

  R_t R;
  R.ring = lds;
  R.red = reinterpret_cast<float*>(lds + D * kG1StageBytes);
  int* tab = reinterpret_cast<int*>(lds + D * kG1StageBytes + NCB * kPRedBytesPerCb);
  R.tab = tab;

  // ---- task table: token row of every column of every task, then each
  // task's expert, dequant scale, row block, first sorted position and first
  // K stage.  The first K stage is a hash of the task index: workgroups that
  // start together would otherwise all read the same 512-byte column of
  // their rows at the same time (measured on E4M3 weights at 32 and 64
  // tokens: 8-9% slower when every task starts at stage 0).
  for (int i = tid; i < ng * CPG; i += 256) {
    const int q = i / CPG, col = i - q * CPG;
    const long long t = w + q * G;
    const int gq = (int)(t / nrb), blk = gq / npb, lc = (gq - blk * npb) * CPG + col;
    int tok = -1;
    if (lc < bm) {
      const int f = a.sorted_ids[(size_t)blk * bm + lc];
      if (f < a.P) tok = f / a.topk;
    }
    tab[q * TW + 5 + col] = tok;
  }
  for (int q = tid; q < ng; q += 256) {
    const long long t = w + q * G;
    const int gq = (int)(t / nrb), blk = gq / npb;
    const int e = a.block_expert[blk];
    float sc = 1.0f;
    if (WT == DT_E4M3) sc = (*a.sx) * a.w13_scale[e];
    tab[q * TW] = e;
    tab[q * TW + 1] = __float_as_int(sc);
    tab[q * TW + 2] = (int)(t - (long long)gq * nrb);
    tab[q * TW + 3] = blk * bm + (gq - blk * npb) * CPG;
    tab[q * TW + 4] = (int)((((unsigned)t * 2654435761u) >> 16) % (unsigned)ns);
  }
  __syncthreads();

  R.w13 = reinterpret_cast<const char*>(a.w13);
  R.xb = reinterpret_cast<const char*>(a.x) + g * 32;
  R.K = K;
  R.N = N;
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

  int cq = 0, ck = 0;  // compute cursor: table row, stage within the task
  float hmax = 0.0f;
  f32x4 accg[NCB], accu[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) accg[cb] = accu[cb] = f32x4{0, 0, 0, 0};

  // end of a task: waves 1..3 leave their partial sums, wave 0 adds them to
  // its own and stores the task's 16 x CPG block of h
  auto finish = [&]() __attribute__((always_inline)) {
    float* red = R.red;
    if (wv > 0) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          red[(((((wv - 1) * 2 + 0) * NCB + cb) * 4 + i) << 6) + lane] = accg[cb][i];
          red[(((((wv - 1) * 2 + 1) * NCB + cb) * 4 + i) << 6) + lane] = accu[cb][i];
        }
    }
    wg_barrier();  // also the stage's closing barrier
    if (wv == 0) {
      const int* row = tab + cq * TW;
      const float scale = __int_as_float(row[1]);
      const int n0 = row[2] * 16;
      const size_t pos0 = (size_t)row[3];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int col = cb * 16 + r16;
        const int t = row[5 + col];
        float h[4], g4[4], u4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float gs = accg[cb][i], us = accu[cb][i];
#pragma unroll
          for (int w2 = 0; w2 < 3; ++w2) {
            gs += red[((((w2 * 2 + 0) * NCB + cb) * 4 + i) << 6) + lane];
            us += red[((((w2 * 2 + 1) * NCB + cb) * 4 + i) << 6) + lane];
          }
          g4[i] = gs * scale;
          u4[i] = us * scale;
          h[i] = silu(g4[i]) * u4[i];
        }
        if (t >= 0) {
          const size_t p = pos0 + col;
          if (a.probe) {
            probe_store(a, p, n0 + 4 * g, g4, u4);
          } else if (WT == DT_E4M3) {
            st16(reinterpret_cast<float*>(a.h) + p * N + n0 + 4 * g,
                 i32x4{__float_as_int(h[0]), __float_as_int(h[1]), __float_as_int(h[2]),
                       __float_as_int(h[3])});
#pragma unroll
            for (int i = 0; i < 4; ++i) hmax = fmaxf(hmax, __builtin_fabsf(h[i]));
          } else {
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.h) + p * N + n0 + 4 * g) =
                make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
          }
        }
      }
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) accg[cb] = accu[cb] = f32x4{0, 0, 0, 0};
    ++cq;
  };

  // Stage p: slot p % D, refilled with stage p + D - 1 while one remains.
  // Whole trips of D stages keep every slot index static (the x fragments
  // live in registers); the tail trip checks p against the total.
  const int total = ng * ns;  // >= ns >= D
  static_for<0, D - 1>([&](auto i) { R.template issue<decltype(i)::value>(); });
  for (int st = 0; st < total; st += D) {
    static_for<0, D>([&](auto i) __attribute__((always_inline)) {
      constexpr int SL = decltype(i)::value;
      const int p = st + SL;
      if (p < total) {
        if (p + D - 1 < total)
          R.template body<SL, true>(accg, accu, g);
        else
          R.template body<SL, false>(accg, accu, g);
        if (++ck == ns) {
          ck = 0;
          finish();
        } else {
          wg_barrier();
        }
      }
    });
  }

  if (WT == DT_E4M3 && wv == 0) {
    hmax = wave_max(hmax);
    if (lane == 0 && hmax > 0.0f) atomicMax(a.hmax_bits, __float_as_uint(hmax));
  }
}

// Launch: WPC workgroups per CU, the task table sized for the longest task
// list a workgroup can get (capacity bound / G, rounded up, plus one).
template <int WT, int NCB, int D, int WPC>
struct G1Ring {
  using R_t = PRing<WT, NCB, D>;
  static int table_rows(const GemmArgs& a) {
    const int bm = a.block_m;
    const long long npb = bm > R_t::CPG ? bm / R_t::CPG : 1;
    const long long cap = (long long)a.P + (long long)min(a.E, a.P) * (bm - 1);
    const long long ntask = (cap + bm - 1) / bm * npb * (a.N / 16);
    const long long G = (long long)WPC * device_cu_count();
    return (int)((ntask + G - 1) / G) + 1;
  }
  static size_t lds(const GemmArgs& a) {
    return (size_t)D * kG1StageBytes + NCB * kPRedBytesPerCb +
           (size_t)table_rows(a) * R_t::TW * sizeof(int);
  }
  static bool fits(const GemmArgs& a) { return lds(a) <= (size_t)160 * 1024 / WPC; }
  static int launch(const GemmArgs& a, hipStream_t st) {
    const size_t bytes = lds(a);
    static size_t attr = 0;  // largest dynamic LDS size enabled so far
    if (bytes > attr) {
      int err = (int)hipFuncSetAttribute((const void*)gemm1_ring_kernel<WT, NCB, D, WPC>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
      if (err) return err;
      attr = bytes;
    }
    hipLaunchKernelGGL((gemm1_ring_kernel<WT, NCB, D, WPC>), dim3(WPC * device_cu_count()),
                       dim3(256), bytes, st, a, table_rows(a));
    return (int)hipGetLastError();
  }
};

// One column block per task for 16-row alignment blocks, two for wider
// ones; two workgroups per CU (measured: one workgroup with an 8-stage ring
// streams 25-40% slower), one when the task table does not leave room for two.
template <int WT, int NCB>
static int g1r_try(const GemmArgs& a, hipStream_t st, bool run) {
  if (G1Ring<WT, NCB, kRingD, 2>::fits(a)) return run ? G1Ring<WT, NCB, kRingD, 2>::launch(a, st) : 0;
  if (G1Ring<WT, NCB, kRingD, 1>::fits(a)) return run ? G1Ring<WT, NCB, kRingD, 1>::launch(a, st) : 0;
  return -1;
}

template <int WT>
static int g1r_dispatch(const GemmArgs& a, hipStream_t st, bool run) {
  return a.block_m <= 16 ? g1r_try<WT, 1>(a, st, run) : g1r_try<WT, 2>(a, st, run);
}

bool gemm1_ring_applies(const GemmArgs& a) {
  if (!((a.wt == DT_BF16 && a.xt == DT_BF16) || (a.wt == DT_E4M3 && a.xt == DT_E4M3)))
    return false;
  const long long row = (long long)a.K * (a.wt == DT_BF16 ? 2 : 1);
  if (row % kRingRowBytes != 0 || row / kRingRowBytes < kRingD || a.N % 16 != 0) return false;
  return (a.wt == DT_E4M3 ? g1r_dispatch<DT_E4M3>(a, nullptr, false)
                          : g1r_dispatch<DT_BF16>(a, nullptr, false)) == 0;
}

int launch_gemm1_ring(const GemmArgs& a, hipStream_t st) {
  return a.wt == DT_E4M3 ? g1r_dispatch<DT_E4M3>(a, st, true) : g1r_dispatch<DT_BF16>(a, st, true);
}

}  // namespace moe

// ===================================================== down GEMM (decode)
//
// Output-stationary down projection with the top-k combine fused, streaming
// w2 through the same kind of ring.  Workgroup = 8 waves and 16 output rows
// n0..n0+15; the stage sequence walks the active experts in id order, for
// each expert its column passes (16*NCB tokens) and its K chunks (1 KiB of
// each of the 16 rows = 8 K-steps, one per wave).  Each wave accumulates its
// K-step's share for the current (expert, pass); on the pass's last chunk it
// multiplies by scale * routing weight and adds into its own LDS accumulator
// [M][16]; the 8 accumulators are summed in a fixed order at the end.  The
// expert table and the per-position (token, weight) table are built in LDS
// before the ring starts, so the steady loop issues no other memory reads
// than the ring's and the h fragments travelling with it.
namespace moe {

constexpr int kG2RingWaves = 8;
constexpr int kG2ChunkBytes = 1024;  // bytes of each w2 row per stage
constexpr int kG2StageBytes = 16 * kPairStride;  // 2 halves x 8 two-row blocks
constexpr int kG2RingMinM = 4;   // M range that takes the down-GEMM ring (measured:
constexpr int kG2RingMaxM = 16;  // faster than the register kernel at T=8, slower at 1, 64)

// (row r < 16, logical byte b < 1024) inside a down-GEMM stage
__device__ __forceinline__ int ring2_off(int r, int b) {
  return ((b >> 9) * 8 + (r >> 1)) * kPairStride + (r & 1) * kRingRowBytes +
         ((b & 511) ^ ((r & 1) << 7));
}

struct G2Table {  // LDS tables of the down-GEMM ring
  int* ek;        // [maxU] expert id
  int* seg;       // [maxU] first sorted position
  int* me;        // [maxU] real pairs
  int* start;     // [maxU + 1] first stage of the expert
  float* sc;      // [maxU] dequant scale of w2 (E4M3) times s_h, else 1
  int* ptok;      // [cap] token of each sorted position (-1: padding)
  float* pwt;     // [cap] routing weight of each sorted position
};

template <int WT, int OT, int NCB, int D>
__global__ __launch_bounds__(512) void gemm2_ring_kernel(GemmArgs a, int maxU, int cap) {
  constexpr int HT = (WT == DT_E4M3) ? DT_E4M3 : DT_BF16;
  constexpr int NI = 2 + 2 * NCB;  // vector-memory instructions per issue
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int M = a.M, K = a.K, N = a.N;
  const int n0 = blockIdx.x * 16;
  constexpr int WB = Family<WT>::kBytes, HB = Family<HT>::kBytes;
  const int nchunk = N * WB / kG2ChunkBytes;

  // ---- LDS carve-up
  char* ring = lds;
  float* acc_lds = reinterpret_cast<float*>(lds + D * kG2StageBytes);  // [8][M][16]
  int* ti = reinterpret_cast<int*>(acc_lds + kG2RingWaves * M * 16);
  G2Table T;
  T.ek = ti;
  T.seg = T.ek + maxU;
  T.me = T.seg + maxU;
  T.start = T.me + maxU;
  T.sc = reinterpret_cast<float*>(T.start + maxU + 1);
  T.ptok = reinterpret_cast<int*>(T.sc + maxU);
  T.pwt = reinterpret_cast<float*>(T.ptok + cap);
  __shared__ int s_U;

  // ---- tables: active experts (wave 0), per-position token/weight (all)
  for (int i = tid; i < kG2RingWaves * M * 16; i += blockDim.x) acc_lds[i] = 0.0f;
  const int npad = *a.num_padded;
  for (int pos = tid; pos < npad; pos += blockDim.x) {
    const int f = a.sorted_ids[pos];
    const bool real = f < a.P;
    T.ptok[pos] = real ? f / a.topk : -1;
    T.pwt[pos] = real ? a.topk_w[f] : 0.0f;
  }
  if (wv == 0) {
    int U = 0;
    for (int base = 0; base < a.E; base += kWave) {
      const int e = base + lane;
      int o0 = 0, o1 = 0;
      if (e < a.E) {
        o0 = a.offsets[e];
        o1 = a.offsets[e + 1];
      }
      const bool act = o1 > o0;
      const uint64_t bal = __ballot(act);
      if (act) {
        const int k = U + __popcll(bal & lanemask_lt(lane));
        T.ek[k] = e;
        T.seg[k] = o0;
        T.me[k] = o1 - o0;  // padded count; trimmed below
      }
      U += __popcll(bal);
    }
    if (lane == 0) s_U = U;
  }
  __syncthreads();
  const int U = s_U;
  // real count = padded count minus the trailing padding positions
  for (int k = tid; k < U; k += blockDim.x) {
    int m = T.me[k];
    const int s0 = T.seg[k];
    while (m > 0 && T.ptok[s0 + m - 1] < 0) --m;
    T.me[k] = m;
    float sc = 1.0f;
    if (WT == DT_E4M3) sc = (*a.sh) * a.w2_scale[T.ek[k]];
    T.sc[k] = sc;
  }
  __syncthreads();
  if (wv == 0) {  // stage starts: prefix sum of npass * nchunk
    int run = 0;
    for (int base = 0; base < U; base += kWave) {
      const int k = base + lane;
      int v = 0;
      if (k < U) v = ((T.me[k] + 16 * NCB - 1) / (16 * NCB)) * nchunk;
      int x = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
      }
      if (k < U) T.start[k] = run + x - v;
      run += __shfl(x, 63, kWave);
    }
    if (lane == 0) T.start[U] = run;
  }
  __syncthreads();
  const int S = T.start[U];

  // ---- per-lane DMA geometry: wave wv issues blocks 2wv, 2wv+1
  const int lrow = lane >> 5;
  const int lb = ((lane & 31) << 4) ^ (lrow << 7);
  int rowo[2], dst[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int bi = 2 * wv + q, rp = bi & 7;  // block bi: half bi >> 3, row pair rp
    rowo[q] = n0 + 2 * rp + lrow;            // w2 row within the expert
    dst[q] = bi * kPairStride;               // block order of ring2_off
  }
  const int hbyte[2] = {((2 * wv) >> 3) * 512 + lb, ((2 * wv + 1) >> 3) * 512 + lb};
  const char* w2 = reinterpret_cast<const char*>(a.w2);
  const char* hq = reinterpret_cast<const char*>(a.hq);

  // cursor over stages: expert k, pass, chunk
  struct Cur {
    int k, pass, chunk;
  };
  auto advance = [&](Cur& c) {
    if (++c.chunk == nchunk) {
      c.chunk = 0;
      ++c.pass;
      if (T.start[c.k] + (c.pass) * nchunk >= T.start[c.k + 1]) {
        c.pass = 0;
        ++c.k;
      }
    }
  };

  Raw<HT> hs[D][NCB];
  auto issue_dma = [&](const Cur& c, int slot) {
    const int e = T.ek[c.k];
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(w2 + ((size_t)e * K + rowo[q]) * N * WB +
                                        (size_t)c.chunk * kG2ChunkBytes + hbyte[q]),
          reinterpret_cast<void*>(ring + slot * kG2StageBytes + dst[q]), 16, 0, kRingAux);
  };
  auto h_src = [&](const Cur& c, int cb) {
    const int col = c.pass * 16 * NCB + cb * 16 + r16;
    const int pos = T.seg[c.k] + (col < T.me[c.k] ? col : 0);
    return hq + (size_t)pos * N * HB + (size_t)c.chunk * kG2ChunkBytes * HB / WB +
           (size_t)(wv * 128 + g * 32) * HB / WB;
  };

  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0, 0, 0, 0};
  float* my = acc_lds + (size_t)wv * M * 16;

  auto compute = [&](const Cur& c, int slot, const Raw<HT>* hx) {
    const char* sb = ring + slot * kG2StageBytes;
    const int o = ring2_off(r16, wv * 128 + g * 32);
    Raw<WT> aw;
    aw.q[0] = ld16(sb + o);
    aw.q[1] = ld16(sb + o + 16);
    const auto A = to_op<WT>(aw);
    const int me = T.me[c.k];
    const int ncb = min(NCB, (me - c.pass * 16 * NCB + 15) / 16);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      if (cb < ncb) acc[cb] = mma(A, to_op<HT>(hx[cb]), acc[cb]);
    if (c.chunk == nchunk - 1) {  // end of this (expert, pass): flush
      const float sc = T.sc[c.k];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int col = c.pass * 16 * NCB + cb * 16 + r16;
        if (cb < ncb && col < me) {
          const int pos = T.seg[c.k] + col;
          const float m = sc * T.pwt[pos];
          float* dd = my + (size_t)T.ptok[pos] * 16 + 4 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i) dd[i] += acc[cb][i] * m;
        }
        acc[cb] = f32x4{0, 0, 0, 0};
      }
    }
  };

  Cur ci{0, 0, 0}, cc{0, 0, 0};
  int issued = 0;
  auto issue = [&](auto slot_c) {  // h fragments + DMA of stage `issued` into ring slot
    constexpr int SLOT = decltype(slot_c)::value;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) hs[SLOT][cb] = load_raw<HT>(h_src(ci, cb));
    issue_dma(ci, SLOT);
    stage_fence();
    advance(ci);
    ++issued;
  };
  if (S >= 2 * D - 1) {
    static_for<0, D - 1>(issue);
    int st = 0;
    for (; st + 2 * D - 2 < S; st += D) {
      static_for<0, D>([&](auto slot_c) {
        constexpr int SLOT = decltype(slot_c)::value;
        issue(std::integral_constant<int, (SLOT + D - 1) % D>{});
        wait_vmcnt<(D - 1) * NI>();
        wg_barrier();
        compute(cc, SLOT, hs[SLOT]);
        advance(cc);
        wg_barrier();
      });
    }
    // remaining stages: those already issued sit in the ring (their h
    // fragments are re-read below), the rest is issued one at a time
    for (; st < S; ++st) {
      if (st >= issued) {
        issue_dma(ci, st % D);
        advance(ci);
        ++issued;
      }
      wait_vmcnt<0>();
      wg_barrier();
      Raw<HT> hx[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) hx[cb] = load_raw<HT>(h_src(cc, cb));
      compute(cc, st % D, hx);
      advance(cc);
      wg_barrier();
    }
  } else {
    for (int st = 0; st < S; ++st) {
      issue_dma(ci, 0);
      advance(ci);
      Raw<HT> hx[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) hx[cb] = load_raw<HT>(h_src(cc, cb));
      wait_vmcnt<0>();
      wg_barrier();
      compute(cc, 0, hx);
      advance(cc);
      wg_barrier();
    }
  }
  __syncthreads();
  for (int i = tid; i < M * 4; i += blockDim.x) {
    const int t = i >> 2, q = (i & 3) * 4;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 0.0f;
      for (int w = 0; w < kG2RingWaves; ++w) s += acc_lds[((size_t)w * M + t) * 16 + q + j];
      v[j] = s;
    }
    if (OT == DT_BF16) {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + (size_t)t * K + n0 + q) =
          make_uint2(pack_bf16x2(v[0], v[1]),
                     pack_bf16x2(v[2], v[3]));
    } else {
      st16(reinterpret_cast<float*>(a.out) + (size_t)t * K + n0 + q,
           i32x4{__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]),
                 __float_as_int(v[3])});
    }
  }
}

constexpr int kG2RingDeep = 6;  // ring depth when the LDS allows it

static size_t g2r_lds(const GemmArgs& a, int maxU, int cap, int D) {
  return (size_t)D * kG2StageBytes + (size_t)kG2RingWaves * a.M * 16 * 4 +
         ((size_t)maxU * 5 + 1) * 4 + (size_t)cap * 8;
}

static int g2r_depth(const GemmArgs& a) {
  const int maxU = min(a.E, a.P);
  const int cap = a.P + maxU * (a.block_m - 1);
  const size_t budget = 160 * 1024 - 256;
  if (g2r_lds(a, maxU, cap, kG2RingDeep) <= budget) return kG2RingDeep;
  if (g2r_lds(a, maxU, cap, kRingD) <= budget) return kRingD;
  return 0;
}

bool gemm2_ring_applies(const GemmArgs& a) {
  if (!(a.wt == DT_BF16 || a.wt == DT_E4M3)) return false;
  if (a.M < kG2RingMinM || a.M > kG2RingMaxM) return false;
  const long long row = (long long)a.N * (a.wt == DT_BF16 ? 2 : 1);
  if (row % kG2ChunkBytes) return false;
  return g2r_depth(a) > 0;
}

template <int WT, int OT, int NCB, int D>
static int g2r_launch(const GemmArgs& a, hipStream_t st) {
  const int maxU = min(a.E, a.P);
  const int cap = a.P + maxU * (a.block_m - 1);
  const size_t lds = g2r_lds(a, maxU, cap, D);
  static size_t attr = 0;  // largest dynamic LDS size enabled so far
  if (lds > attr) {
    int err = (int)hipFuncSetAttribute((const void*)gemm2_ring_kernel<WT, OT, NCB, D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err) return err;
    attr = lds;
  }
  hipLaunchKernelGGL((gemm2_ring_kernel<WT, OT, NCB, D>), dim3(a.K / 16), dim3(512), lds, st, a,
                     maxU, cap);
  return (int)hipGetLastError();
}

template <int WT, int OT, int NCB>
static int g2r_depth_dispatch(const GemmArgs& a, hipStream_t st) {
  return g2r_depth(a) == kG2RingDeep ? g2r_launch<WT, OT, NCB, kG2RingDeep>(a, st)
                                     : g2r_launch<WT, OT, NCB, kRingD>(a, st);
}

int launch_gemm2_ring(const GemmArgs& a, hipStream_t st) {
  const int ncb = min((min(a.M, kStreamMaxM) + 15) / 16, kRingNcbMax);
#define G2R(W, O)                                                                  \
  return ncb <= 1 ? g2r_depth_dispatch<W, O, 1>(a, st) : g2r_depth_dispatch<W, O, 2>(a, st);
  if (a.wt == DT_E4M3) {
    if (a.ot == DT_BF16) G2R(DT_E4M3, DT_BF16) else G2R(DT_E4M3, DT_F32)
  }
  if (a.ot == DT_BF16) G2R(DT_BF16, DT_BF16) else G2R(DT_BF16, DT_F32)
#undef G2R
}

}  // namespace moe
