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
// Workgroup: 4 waves, 16 gate + 16 up rows of one active expert; every stage
// is 512 bytes of each of the 32 rows (4 K-steps), one step per wave.  Each
// wave keeps its own x fragments of the kRingD - 1 stages in flight in
// registers, issued together with the stage's DMA so that a single in-order
// vmcnt wait covers both.
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

// NRB row blocks per workgroup (16 gate + 16 up rows each) go through the
// ring one after the other: stage p < ns is row block 0's K stage p, stage
// ns + k row block 1's stage k.  More stages per workgroup amortise the
// ring's fill and drain (for E4M3 a row block alone is only 8 stages).
template <int WT, int NCB, int NRB>
struct G1Ring {
  static constexpr int D = kRingD;
  static constexpr int SB = 128;              // bytes per K-step of a row (both families)
  static constexpr int NI = 4 + 2 * NCB;      // vector-memory instructions per issue
  char* lds;
  const char* src[4];   // this lane's DMA source per block (stage 0, row block 0)
  int dst[4];           // LDS offset of each of this wave's blocks
  const char* xr[NCB];  // this lane's x row (+ lane-group offset)
  Raw<WT> xs[D][NCB];
  int wv;
  int ns;               // stages of one row block
  size_t rbstride;      // bytes from one row block's rows to the next one's

  template <int SLOT>
  __device__ __forceinline__ void issue(int p) {
    const int rb = (NRB > 1 && p >= ns) ? 1 : 0;
    const int k = p - rb * ns;  // K stage within the row block
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      xs[SLOT][cb] = load_raw<WT>(xr[cb] + (size_t)(k * 4 + wv) * SB);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(src[q] + rb * rbstride + (size_t)k * kRingRowBytes),
          reinterpret_cast<void*>(lds + SLOT * kG1StageBytes + dst[q]), 16, 0, kRingAux);
    stage_fence();
  }

  // One stage: ISSUE = 1 refills the ring with stage st + D - 1 first (steady
  // state, every earlier stage issued the same instruction count, so the
  // in-order vmcnt of (D-1) issues is exact); ISSUE = 0 drains the ring.
  template <int SLOT, bool ISSUE>
  __device__ __forceinline__ void body(int st, int ncb, int r16, int g, f32x4 accg[NCB],
                                       f32x4 accu[NCB]) {
    if constexpr (ISSUE) {
      issue<(SLOT + D - 1) % D>(st + D - 1);
      wait_vmcnt<(D - 1) * NI>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();
    const char* sb = lds + SLOT * kG1StageBytes;
    const int b = wv * SB + g * 32;
    Raw<WT> ag, au;
    const int og = ring_off(r16, b), ou = ring_off(16 + r16, b);
    ag.q[0] = ld16(sb + og);
    ag.q[1] = ld16(sb + og + 16);
    au.q[0] = ld16(sb + ou);
    au.q[1] = ld16(sb + ou + 16);
    auto A = to_op<WT>(ag);
    auto U = to_op<WT>(au);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      if (cb < ncb) {
        auto X = to_op<WT>(xs[SLOT][cb]);
        accg[cb] = mma(A, X, accg[cb]);
        accu[cb] = mma(U, X, accu[cb]);
      }
    }
    wg_barrier();
  }
};

template <int WT, int NCB, int NRB>
__global__ __launch_bounds__(256, 2) void gemm1_ring_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int D = kRingD;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;

  const int e = nth_active_expert(a.offsets, a.E, blockIdx.y);
  if (e < 0) return;  // uniform over the workgroup
  const int seg0 = a.offsets[e], seg1 = a.offsets[e + 1];
  const int me = segment_count(a.sorted_ids, seg0, seg1, a.P);
  const int n0 = blockIdx.x * 16 * NRB;
  const int K = a.K, N = a.N;
  constexpr int WB = Family<WT>::kBytes;
  const int ns = K * WB / kRingRowBytes;

  G1Ring<WT, NCB, NRB> R;
  R.lds = lds;
  R.wv = wv;
  R.ns = ns;
  R.rbstride = (size_t)16 * K * WB;
  const char* w13 = reinterpret_cast<const char*>(a.w13);
  {
    const int lrow = lane >> 5;
    const int lb = ((lane & 31) << 4) ^ (lrow << 7);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int blk = 4 * wv + q;
      const int r = 2 * blk + lrow;
      const int grow = (r < 16) ? (n0 + r) : (N + n0 + r - 16);
      R.src[q] = w13 + ((size_t)e * 2 * N + grow) * K * WB + lb;
      R.dst[q] = blk * kPairStride;
    }
  }
  const char* xb = reinterpret_cast<const char*>(a.x) + g * 32;

  float scale = 1.0f;
  if (WT == DT_E4M3) scale = (*a.sx) * a.w13_scale[e];
  float hmax = 0.0f;
  float* red = reinterpret_cast<float*>(lds);  // reused after the ring drains

  for (int c0 = 0; c0 < me; c0 += 16 * NCB) {
    const int ncb = min(NCB, (me - c0 + 15) / 16);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int col = c0 + cb * 16 + r16;
      const int f = a.sorted_ids[seg0 + (col < me ? col : 0)];
      R.xr[cb] = xb + (size_t)(f / a.topk) * K * WB;
    }
    f32x4 accg[NRB][NCB], accu[NRB][NCB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) accg[rb][cb] = accu[rb][cb] = f32x4{0, 0, 0, 0};
    // stage s of the sequence: slot SL, refill (IS) or drain; row block 1's
    // stages accumulate into its own registers
    auto stage = [&](auto slot, auto is, int s) {
      constexpr int SL = decltype(slot)::value;
      constexpr bool IS = decltype(is)::value;
      if (NRB == 1 || s < ns)
        R.template body<SL, IS>(s, ncb, r16, g, accg[0], accu[0]);
      else
        R.template body<SL, IS>(s, ncb, r16, g, accg[NRB - 1], accu[NRB - 1]);
    };
    using Refill = std::true_type;
    using Drain = std::false_type;
    const int total = NRB * ns;

    // prologue: stages 0 .. D - 2
    static_for<0, D - 1>([&](auto i) { R.template issue<decltype(i)::value>(decltype(i)::value); });
    // steady state: whole trips of D stages that all refill (total >= D)
    const int n_issue = total - (D - 1);  // stages that refill the ring
    int st = 0;
    for (; st + D <= n_issue; st += D)
      static_for<0, D>([&](auto i) { stage(i, Refill{}, st + decltype(i)::value); });
    // the last n_issue % D refilling stages, then D - 1 draining ones; slot =
    // stage % D is static in every branch
    const int rem = n_issue - st;  // 0 .. D - 1
    static_for<0, D>([&](auto rr) {
      constexpr int RR = decltype(rr)::value;
      if (rem == RR) {
        static_for<0, RR>([&](auto i) { stage(i, Refill{}, st + decltype(i)::value); });
        static_for<0, D - 1>([&](auto j) {
          constexpr int J = decltype(j)::value;
          stage(std::integral_constant<int, (RR + J) % D>{}, Drain{}, st + RR + J);
        });
      }
    });

    // reduce the 4 K-slices of each row block (the ring is drained: every
    // body ended with a barrier)
    static_for<0, NRB>([&](auto rbc) {
    constexpr int RB = decltype(rbc)::value;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red[((((wv * 2 + 0) * NCB + cb) * 4 + i) << 6) + lane] = accg[RB][cb][i];
        red[((((wv * 2 + 1) * NCB + cb) * 4 + i) << 6) + lane] = accu[RB][cb][i];
      }
    __syncthreads();
    for (int cb = wv; cb < ncb; cb += 4) {
      const int col = c0 + cb * 16 + r16;
      float h[4], g4[4], u4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          gs += red[((((w * 2 + 0) * NCB + cb) * 4 + i) << 6) + lane];
          us += red[((((w * 2 + 1) * NCB + cb) * 4 + i) << 6) + lane];
        }
        g4[i] = gs * scale;
        u4[i] = us * scale;
        h[i] = silu(g4[i]) * u4[i];
      }
      if (a.probe) {
        if (col < me) probe_store(a, (size_t)(seg0 + col), n0 + 16 * RB + 4 * g, g4, u4);
      } else if (col < me) {
        const size_t idx = (size_t)(seg0 + col) * N + n0 + 16 * RB + 4 * g;
        if (WT == DT_E4M3) {
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
    __syncthreads();  // red aliases the ring: drain before it is reused
    });
  }
  if (WT == DT_E4M3) {
    hmax = wave_max(hmax);
    if (lane == 0 && hmax > 0.0f) atomicMax(a.hmax_bits, __float_as_uint(hmax));
  }
}

bool gemm1_ring_applies(const GemmArgs& a) {
  if (!((a.wt == DT_BF16 && a.xt == DT_BF16) || (a.wt == DT_E4M3 && a.xt == DT_E4M3)))
    return false;
  const long long row = (long long)a.K * (a.wt == DT_BF16 ? 2 : 1);
  return row % kRingRowBytes == 0 && row / kRingRowBytes >= kRingD;
}

template <int WT, int NCB, int NRB>
static int g1r_launch(const GemmArgs& a, hipStream_t st) {
  const size_t ring = (size_t)kRingD * kG1StageBytes;
  const size_t red = (size_t)4 * 2 * NCB * 4 * kWave * sizeof(float);
  const size_t lds = ring > red ? ring : red;
  static bool attr = false;
  if (!attr) {
    int err = (int)hipFuncSetAttribute((const void*)gemm1_ring_kernel<WT, NCB, NRB>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err) return err;
    attr = true;
  }
  dim3 grid(a.N / (16 * NRB), min(a.E, a.P));
  hipLaunchKernelGGL((gemm1_ring_kernel<WT, NCB, NRB>), grid, dim3(256), lds, st, a);
  return (int)hipGetLastError();
}

// Two row blocks per workgroup for E4M3 with one token column block (half
// the bytes per row, so one row block is too short a stream; measured 5-7%
// faster at T = 1-16).  With two column blocks the second row block's
// accumulators no longer fit two workgroups per CU without spilling, which
// costs more than it gains, so bf16 and wider batches keep one.
template <int WT>
static int g1r_dispatch(const GemmArgs& a, hipStream_t st, int ncb) {
  if constexpr (WT == DT_E4M3) {
    if (ncb <= 1 && a.N % 32 == 0) return g1r_launch<WT, 1, 2>(a, st);
  }
  return ncb <= 1 ? g1r_launch<WT, 1, 1>(a, st) : g1r_launch<WT, 2, 1>(a, st);
}

int launch_gemm1_ring(const GemmArgs& a, hipStream_t st) {
  const int ncb = min((min(a.M, kStreamMaxM) + 15) / 16, kRingNcbMax);
  return a.wt == DT_E4M3 ? g1r_dispatch<DT_E4M3>(a, st, ncb) : g1r_dispatch<DT_BF16>(a, st, ncb);
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
