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
// Workgroup barrier without the fence of __syncthreads (which would also wait
// for the ring's outstanding loads); the empty asm keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int WT, int NCB>
struct G1Ring {
  static constexpr int D = kRingD;
  static constexpr int SB = 128;              // bytes per K-step of a row (both families)
  static constexpr int NI = 4 + 2 * NCB;      // vector-memory instructions per issue
  char* lds;
  const char* src[4];   // this lane's DMA source per block (stage 0)
  int dst[4];           // LDS offset of each of this wave's blocks
  const char* xr[NCB];  // this lane's x row (+ lane-group offset)
  Raw<WT> xs[D][NCB];
  int wv;

  template <int SLOT>
  __device__ __forceinline__ void issue(int p) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      xs[SLOT][cb] = load_raw<WT>(xr[cb] + (size_t)(p * 4 + wv) * SB);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(src[q] + (size_t)p * kRingRowBytes),
          reinterpret_cast<void*>(lds + SLOT * kG1StageBytes + dst[q]), 16, 0, kRingAux);
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

template <int WT, int NCB>
__global__ __launch_bounds__(256) void gemm1_ring_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int D = kRingD;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;

  const int e = nth_active_expert(a.offsets, a.E, blockIdx.y);
  if (e < 0) return;  // uniform over the workgroup
  const int seg0 = a.offsets[e], seg1 = a.offsets[e + 1];
  const int me = segment_count(a.sorted_ids, seg0, seg1, a.P);
  const int n0 = blockIdx.x * 16;
  const int K = a.K, N = a.N;
  constexpr int WB = Family<WT>::kBytes;
  const int ns = K * WB / kRingRowBytes;

  G1Ring<WT, NCB> R;
  R.lds = lds;
  R.wv = wv;
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
    f32x4 accg[NCB], accu[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) accg[cb] = accu[cb] = f32x4{0, 0, 0, 0};

    static_assert(D == 4, "prologue and drain written for four stages");
    R.template issue<0>(0);
    R.template issue<1>(1);
    R.template issue<2>(2);
    // steady state: whole trips of D stages that all refill (ns >= D)
    const int n_issue = ns - (D - 1);  // stages that refill the ring
    int st = 0;
    for (; st + D <= n_issue; st += D) {
      R.template body<0, true>(st + 0, ncb, r16, g, accg, accu);
      R.template body<1, true>(st + 1, ncb, r16, g, accg, accu);
      R.template body<2, true>(st + 2, ncb, r16, g, accg, accu);
      R.template body<3, true>(st + 3, ncb, r16, g, accg, accu);
    }
    // the last n_issue % D refilling stages, then D - 1 draining ones; slot =
    // stage % D is static in every branch
    const int rem = n_issue - st;  // 0..3
    if (rem == 0) {
      R.template body<0, false>(st + 0, ncb, r16, g, accg, accu);
      R.template body<1, false>(st + 1, ncb, r16, g, accg, accu);
      R.template body<2, false>(st + 2, ncb, r16, g, accg, accu);
    } else if (rem == 1) {
      R.template body<0, true>(st + 0, ncb, r16, g, accg, accu);
      R.template body<1, false>(st + 1, ncb, r16, g, accg, accu);
      R.template body<2, false>(st + 2, ncb, r16, g, accg, accu);
      R.template body<3, false>(st + 3, ncb, r16, g, accg, accu);
    } else if (rem == 2) {
      R.template body<0, true>(st + 0, ncb, r16, g, accg, accu);
      R.template body<1, true>(st + 1, ncb, r16, g, accg, accu);
      R.template body<2, false>(st + 2, ncb, r16, g, accg, accu);
      R.template body<3, false>(st + 3, ncb, r16, g, accg, accu);
      R.template body<0, false>(st + 4, ncb, r16, g, accg, accu);
    } else {
      R.template body<0, true>(st + 0, ncb, r16, g, accg, accu);
      R.template body<1, true>(st + 1, ncb, r16, g, accg, accu);
      R.template body<2, true>(st + 2, ncb, r16, g, accg, accu);
      R.template body<3, false>(st + 3, ncb, r16, g, accg, accu);
      R.template body<0, false>(st + 4, ncb, r16, g, accg, accu);
      R.template body<1, false>(st + 5, ncb, r16, g, accg, accu);
    }

    // reduce the 4 K-slices (the ring is drained: every body ended with a barrier)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red[((((wv * 2 + 0) * NCB + cb) * 4 + i) << 6) + lane] = accg[cb][i];
        red[((((wv * 2 + 1) * NCB + cb) * 4 + i) << 6) + lane] = accu[cb][i];
      }
    __syncthreads();
    for (int cb = wv; cb < ncb; cb += 4) {
      const int col = c0 + cb * 16 + r16;
      float h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          gs += red[((((w * 2 + 0) * NCB + cb) * 4 + i) << 6) + lane];
          us += red[((((w * 2 + 1) * NCB + cb) * 4 + i) << 6) + lane];
        }
        h[i] = silu(gs * scale) * (us * scale);
      }
      if (col < me) {
        const size_t idx = (size_t)(seg0 + col) * N + n0 + 4 * g;
        if (WT == DT_E4M3) {
          st16(reinterpret_cast<float*>(a.h) + idx,
               i32x4{__float_as_int(h[0]), __float_as_int(h[1]), __float_as_int(h[2]),
                     __float_as_int(h[3])});
#pragma unroll
          for (int i = 0; i < 4; ++i) hmax = fmaxf(hmax, __builtin_fabsf(h[i]));
        } else {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.h) + idx) =
              make_uint2(f32_to_bf16_bits(h[0]) | (f32_to_bf16_bits(h[1]) << 16),
                         f32_to_bf16_bits(h[2]) | (f32_to_bf16_bits(h[3]) << 16));
        }
      }
    }
    __syncthreads();  // red aliases the ring: drain before the next pass refills it
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

template <int WT, int NCB>
static int g1r_launch(const GemmArgs& a, hipStream_t st) {
  const size_t ring = (size_t)kRingD * kG1StageBytes;
  const size_t red = (size_t)4 * 2 * NCB * 4 * kWave * sizeof(float);
  const size_t lds = ring > red ? ring : red;
  static bool attr = false;
  if (!attr) {
    int err = (int)hipFuncSetAttribute((const void*)gemm1_ring_kernel<WT, NCB>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err) return err;
    attr = true;
  }
  dim3 grid(a.N / 16, min(a.E, a.P));
  hipLaunchKernelGGL((gemm1_ring_kernel<WT, NCB>), grid, dim3(256), lds, st, a);
  return (int)hipGetLastError();
}

int launch_gemm1_ring(const GemmArgs& a, hipStream_t st) {
  const int ncb = min((min(a.M, kStreamMaxM) + 15) / 16, kRingNcbMax);
  if (a.wt == DT_E4M3)
    return ncb <= 1 ? g1r_launch<DT_E4M3, 1>(a, st) : g1r_launch<DT_E4M3, 2>(a, st);
  return ncb <= 1 ? g1r_launch<DT_BF16, 1>(a, st) : g1r_launch<DT_BF16, 2>(a, st);
}

}  // namespace moe
