// ring.hip -- launchers of the decode expert GEMMs (gate/up and down) on the
// LDS weight ring of ring.hpp: one launch of WPC workgroups per CU each.
#include "ring.hpp"

namespace moe {

template <int WT, int NCB, int D, int WPC, bool G1>
__global__ __launch_bounds__(kRingThreads, WPC) void ring_gemm_kernel(GemmArgs a, int GT) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  if constexpr (NCB == 0) {
    int base;
    const int npair = pair_scan(a, reinterpret_cast<int*>(lds + D * kG1StageBytes), base);
    const int nb = *a.num_padded / a.block_m;
    if (kPairGain * (nb - npair) >= nb && npair < nb) {
      // the heads sit in the ring's space, free until the first load is issued
      int* heads = reinterpret_cast<int*>(lds);
      pair_heads(a, base, heads);
      ring_run<WT, 2, D - 1, G1>(a, GT, lds, heads, npair);
    } else {
      ring_run<WT, 1, D, G1>(a, GT, lds, nullptr, 0);
    }
  } else {
    ring_run<WT, NCB, D, G1>(a, GT, lds, nullptr, 0);
  }
}

// Launch: WPC workgroups per CU (sizes in ring.hpp).
template <int WT, int NCB, int D, int WPC, bool G1>
struct RingGemm : RingSize<WT, NCB, D, WPC, G1> {
  using RingSize<WT, NCB, D, WPC, G1>::lds;
  using RingSize<WT, NCB, D, WPC, G1>::table_rows;
  static int launch(const GemmArgs& a, hipStream_t st) {
    const size_t bytes = lds(a);
    // the limit is set once per device to the most any launch may ask (fits())
    static OncePerDevice attr;
    const int err = attr.run([] {
      return (int)hipFuncSetAttribute((const void*)ring_gemm_kernel<WT, NCB, D, WPC, G1>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                      160 * 1024 / WPC);
    });
    if (err) return err;
    hipLaunchKernelGGL((ring_gemm_kernel<WT, NCB, D, WPC, G1>), dim3(WPC * device_cu_count()),
                       dim3(kRingThreads), bytes, st, a, table_rows(a));
    return (int)hipGetLastError();
  }
};

// Two workgroups per CU (measured: one workgroup with an 8-stage ring
// streams 25-40% slower), one when the task table does not leave room for
// two.  run = false only asks whether a launch would fit (0) or not (-1).
template <int WT, int NCB, bool G1>
static int ring_try(const GemmArgs& a, hipStream_t st, bool run) {
  if (RingGemm<WT, NCB, kRingD, 2, G1>::fits(a))
    return run ? RingGemm<WT, NCB, kRingD, 2, G1>::launch(a, st) : 0;
  if (RingGemm<WT, NCB, kRingD, 1, G1>::fits(a))
    return run ? RingGemm<WT, NCB, kRingD, 1, G1>::launch(a, st) : 0;
  return -1;
}

// 16-row alignment blocks: NCB = 0 (one- or two-block column groups, chosen
// by the kernel) where the pairing scan covers E and the group heads fit in
// the ring's space, else one block per group.
constexpr bool kPairG1 = true;
constexpr bool kPairG2 = true;

template <bool G1>
static int ring_dispatch(const GemmArgs& a, hipStream_t st, bool run) {
  if (a.block_m > 16)
    return a.wt == DT_E4M3 ? ring_try<DT_E4M3, 2, G1>(a, st, run) : ring_try<DT_BF16, 2, G1>(a, st, run);
  // pairing needs an expert with two 16-row blocks, so more than 16 pairs
  if ((G1 ? kPairG1 : kPairG2) && a.P > 16 && ring_pair_fits(a))
    return a.wt == DT_E4M3 ? ring_try<DT_E4M3, 0, G1>(a, st, run) : ring_try<DT_BF16, 0, G1>(a, st, run);
  return a.wt == DT_E4M3 ? ring_try<DT_E4M3, 1, G1>(a, st, run) : ring_try<DT_BF16, 1, G1>(a, st, run);
}

bool gemm1_ring_applies(const GemmArgs& a) {
  if (!((a.wt == DT_BF16 && a.xt == DT_BF16) || (a.wt == DT_E4M3 && a.xt == DT_E4M3)))
    return false;
  if (!ring_rows(a, a.K) || a.N % 16 != 0 || a.M >= 255) return false;  // token rows in bytes
  return ring_dispatch<true>(a, nullptr, false) == 0;
}

int launch_gemm1_ring(const GemmArgs& a, hipStream_t st) { return ring_dispatch<true>(a, st, true); }

// Below 4 tokens the down GEMM keeps the streaming kernel with the combine
// fused (measured at 1 token: the ring plus a combine launch is 3 us slower).
constexpr int kG2RingMinM = 4;

bool gemm2_ring_applies(const GemmArgs& a) {
  if (!(a.wt == DT_BF16 || a.wt == DT_E4M3) || !(a.ot == DT_BF16 || a.ot == DT_F32)) return false;
  if (a.M < kG2RingMinM) return false;
  if (!ring_rows(a, a.N) || a.K % 32 != 0) return false;
  return ring_dispatch<false>(a, nullptr, false) == 0;
}

int launch_gemm2_ring(const GemmArgs& a, hipStream_t st) { return ring_dispatch<false>(a, st, true); }

}  // namespace moe
