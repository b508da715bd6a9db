// prefill.hip -- expert GEMMs for large token counts (prefill), where every
// active expert has hundreds of token rows and the products are dense
// contractions bound by the matrix cores.
//
// Same grouped problem as the decode kernels ("Amazon SageMaker AI 上的
// Mixture-of-Experts 内核工程优化", introduction: tokens bucketed per expert,
// one GEMM per expert), on a macro tile of 256 weight rows x 128 token rows:
// the token rows are one alignment block of one expert (gathered through the
// sorted pair list), the weight rows are Bᵀ rows of that expert, so the
// product is computed as Bᵀ·Aᵀ with the weights on the MFMA row operand, as
// in the decode kernels.
//
// Both operands are staged through a three-stage LDS ring filled by
// direct-to-LDS loads (global_load_lds_dwordx4): each stage holds 128 bytes
// of K of every row (64 bf16 or 128 E4M3 values), 48 KiB in all.  A wave
// instruction moves 8 rows x 128 bytes; the source addresses, not the LDS
// writes, are permuted so that row r's 16-byte column c lands at physical
// column (c + r) mod 8.  Lane group g of an MFMA fragment takes the logical
// columns g and g + 4 (any K order serves, as long as both operands use the
// same one).  Measured on MI355X with ds_read_b128, this pairing of column
// assignment and rotation reads at the linear-access rate, while the
// assignment 2g, 2g + 1 is two-way bank-conflicted under every swizzle tried.
//
// Workgroup: 4 waves (one per SIMD) as 2 (weight rows) x 2 (tokens); each
// wave owns a 128 x 64 sub-tile = 8 x 4 MFMA tiles of 16 x 16, whose
// accumulators live in the accumulation registers, and double-buffers its
// operand fragments in registers.  For the gate/up product the 128 rows of a
// wave are 64 gate rows followed by the 64 up rows of the same intermediate
// columns, so SiLU(gate) * up is formed in registers.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kPfRows = 256;                          // weight rows per tile
constexpr int kPfTok = 128;                           // token rows per tile
constexpr int kPfChunk = 128;                         // bytes of K per row and stage
constexpr int kPfStages = 3;
constexpr int kPfWBytes = kPfRows * kPfChunk;         // 32 KiB
constexpr int kPfXBytes = kPfTok * kPfChunk;          // 16 KiB
constexpr int kPfStageBytes = kPfWBytes + kPfXBytes;  // 48 KiB
constexpr int kPfLdsBytes = kPfStages * kPfStageBytes;
constexpr int kPfThreads = 256;
constexpr int kPfWaves = kPfThreads / kWave;
constexpr int kPfWInstr = kPfWBytes / 1024 / kPfWaves;  // 8 DMA instructions per wave
constexpr int kPfXInstr = kPfXBytes / 1024 / kPfWaves;  // 4
constexpr int kPfTA = 8;  // 16-row weight tiles per wave
constexpr int kPfTB = 4;  // 16-row token tiles per wave
constexpr int kPfNI = kPfWInstr + kPfXInstr;
constexpr int kPfAux = 0;  // cache policy of the DMA (operands are re-read by other tiles)

// LDS offset of logical 16-byte column c of row r (see the header), and the
// logical column that lands at physical column p of row r.
__device__ __forceinline__ int pf_off(int r, int c) { return r * kPfChunk + (((c + r) & 7) << 4); }
__device__ __forceinline__ int pf_logical(int r, int p) { return (p - r) & 7; }

template <int N>
__device__ __forceinline__ void pf_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Workgroup barrier that first lets this wave's LDS reads complete (so no
// wave refills a stage another wave is still reading) but, unlike
// __syncthreads, does not wait for the ring's outstanding loads.
__device__ __forceinline__ void pf_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// XCD-aware task order: the hardware deals consecutive workgroup ids
// round-robin over the 8 XCDs; each XCD is given a contiguous range of
// (weight tile, token block) tasks, token block fastest, so that the blocks
// that share one expert's weight tile run together on one L2.
__device__ __forceinline__ void pf_task(int& nt, int& mb) {
  const int nblk = gridDim.y, ntiles = gridDim.x;
  const int total = nblk * ntiles;
  const int lin = blockIdx.y * ntiles + blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = lin % 8, k = lin / 8;
  const int task = xcd * per + min(xcd, rem) + k;
  nt = task / nblk, mb = task % nblk;
}

// G1 = true: gate/up product + SiLU * up -> h.  G1 = false: down product
// times the routing weight -> y (one row per sorted position).
template <int T, bool G1>
__global__ __launch_bounds__(kPfThreads) void pf_gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int nt, mb;
  pf_task(nt, mb);
  if (mb * kPfTok >= *a.num_padded) return;  // uniform: past the last block
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int wr = wv >> 1, wc = wv & 1;
  const int e = a.block_expert[(mb * kPfTok) / a.block_m];
  const int Kd = G1 ? a.K : a.N;  // contraction length
  constexpr int EB = Family<T>::kBytes;
  const size_t rowb = (size_t)Kd * EB;
  const int nchunks = (int)(rowb / kPfChunk);

  // Per-lane DMA sources of chunk 0.  A wave's 8 weight instructions cover
  // 64 consecutive tile rows, which are 64 consecutive rows of the weight
  // matrix (gate or up block for the gate/up product); the rotation of row r
  // only depends on r mod 8, so one lane offset serves all of them.
  const int lrow = lane >> 3, pcol = lane & 7;
  const char* wbase;
  {
    const int r0 = 64 * wv;  // first tile row of this wave's weight DMA
    size_t grow0;
    if (G1) {
      const int h0 = nt * 128 + 64 * (r0 >> 7);  // first intermediate column
      grow0 = (size_t)e * 2 * a.N + ((r0 & 127) < 64 ? h0 : a.N + h0);
      wbase = reinterpret_cast<const char*>(a.w13) + grow0 * rowb;
    } else {
      grow0 = (size_t)e * a.K + nt * kPfRows + r0;
      wbase = reinterpret_cast<const char*>(a.w2) + grow0 * rowb;
    }
  }
  const uint32_t woff = (uint32_t)(lrow * rowb) + (uint32_t)(pf_logical(lrow, pcol) * 16);
  const char* xsrc[kPfXInstr];
#pragma unroll
  for (int q = 0; q < kPfXInstr; ++q) {
    const int r = 8 * (wv * kPfXInstr + q) + lrow;  // token row 0..127
    const int c = pf_logical(r, pcol);
    const int pos = mb * kPfTok + r;
    if (G1) {
      int f = a.sorted_ids[pos];
      if (f >= a.P) f = 0;  // padding row: any valid row, never stored
      xsrc[q] = reinterpret_cast<const char*>(a.x) + (size_t)(f / a.topk) * rowb + c * 16;
    } else {
      xsrc[q] = reinterpret_cast<const char*>(a.hq) + (size_t)pos * rowb + c * 16;
    }
  }

  auto issue = [&](int chunk, int slot) {
    char* sb = lds + slot * kPfStageBytes;
    const size_t off = (size_t)chunk * kPfChunk;
#pragma unroll
    for (int q = 0; q < kPfWInstr; ++q)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(wbase + off + (size_t)(8 * q) * rowb + woff),
          reinterpret_cast<void*>(sb + (wv * kPfWInstr + q) * 1024), 16, 0, kPfAux);
#pragma unroll
    for (int q = 0; q < kPfXInstr; ++q)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(xsrc[q] + off),
          reinterpret_cast<void*>(sb + kPfWBytes + (wv * kPfXInstr + q) * 1024), 16, 0, kPfAux);
  };

  f32x4 acc[kPfTA][kPfTB];
#pragma unroll
  for (int i = 0; i < kPfTA; ++i)
#pragma unroll
    for (int j = 0; j < kPfTB; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  // LDS offsets of this lane's fragments (logical columns g and g + 4); tile
  // i adds i * 16 rows = i * 2048 bytes (the rotation repeats every 8 rows)
  int aoff[2], boff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    aoff[h] = pf_off(128 * wr + r16, g + 4 * h);
    boff[h] = kPfWBytes + pf_off(64 * wc + r16, g + 4 * h);
  }

  // Fragments of chunk c are read from LDS right after the barrier that
  // publishes it and consumed one iteration later, so the MFMAs of chunk c - 1
  // cover the LDS latency of chunk c; the DMA runs two chunks ahead.
  auto load_frags = [&](int slot, Raw<T> (&A)[kPfTA], Raw<T> (&B)[kPfTB]) {
    const char* sb = lds + slot * kPfStageBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < kPfTB; ++j) B[j].q[h] = ld16(sb + boff[h] + j * 16 * kPfChunk);
#pragma unroll
      for (int i = 0; i < kPfTA; ++i) A[i].q[h] = ld16(sb + aoff[h] + i * 16 * kPfChunk);
    }
  };
  auto compute = [&](const Raw<T> (&A)[kPfTA], const Raw<T> (&B)[kPfTB]) {
#pragma unroll
    for (int i = 0; i < kPfTA; ++i) {
      auto Ai = to_op<T>(A[i]);
#pragma unroll
      for (int j = 0; j < kPfTB; ++j) acc[i][j] = mma(Ai, to_op<T>(B[j]), acc[i][j]);
    }
  };
  // Iteration c (c + 1 < nchunks): wait for chunk c + 1, barrier (chunk c + 1
  // visible; every wave holds chunk c's fragments, so stage c % 3 is free),
  // refill that stage with chunk c + 3, read chunk c + 1's fragments, multiply
  // chunk c.  The accumulators flow through straight-line code only (no
  // branch around an MFMA), so they keep their registers across iterations.
  auto step = [&](int c, Raw<T> (&Ac)[kPfTA], Raw<T> (&Bc)[kPfTB], Raw<T> (&An)[kPfTA],
                  Raw<T> (&Bn)[kPfTB]) {
    if (c + 2 < nchunks)
      pf_wait_vmcnt<kPfNI>();
    else
      pf_wait_vmcnt<0>();
    pf_barrier();
    if (c + 3 < nchunks) issue(c + 3, c % 3);
    load_frags((c + 1) % 3, An, Bn);
    compute(Ac, Bc);
  };

  issue(0, 0);
  if (nchunks > 1) issue(1, 1);
  if (nchunks > 2) issue(2, 2);
  if (nchunks > 2)
    pf_wait_vmcnt<2 * kPfNI>();
  else if (nchunks > 1)
    pf_wait_vmcnt<kPfNI>();
  else
    pf_wait_vmcnt<0>();
  pf_barrier();
  Raw<T> A0[kPfTA], B0[kPfTB], A1[kPfTA], B1[kPfTB];
  load_frags(0, A0, B0);
  int c = 0;
  for (; c + 2 < nchunks; c += 2) {
    step(c, A0, B0, A1, B1);
    step(c + 1, A1, B1, A0, B0);
  }
  if (c + 1 < nchunks) {  // two chunks left
    step(c, A0, B0, A1, B1);
    compute(A1, B1);
  } else {  // one chunk left
    compute(A0, B0);
  }

  if constexpr (G1) {
    float scale = 1.0f;
    if (T == DT_E4M3) scale = (*a.sx) * a.w13_scale[e];
    float hmax = 0.0f;
#pragma unroll
    for (int j = 0; j < kPfTB; ++j) {
      const int pos = mb * kPfTok + 64 * wc + 16 * j + r16;
      if (a.sorted_ids[pos] < a.P) {
#pragma unroll
        for (int i = 0; i < kPfTA / 2; ++i) {
          float h[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            h[t] = silu(acc[i][j][t] * scale) * (acc[i + kPfTA / 2][j][t] * scale);
          const size_t idx = (size_t)pos * a.N + nt * 128 + 64 * wr + 16 * i + 4 * g;
          if (T == DT_E4M3) {
            st16(reinterpret_cast<float*>(a.h) + idx,
                 i32x4{__float_as_int(h[0]), __float_as_int(h[1]), __float_as_int(h[2]),
                       __float_as_int(h[3])});
#pragma unroll
            for (int t = 0; t < 4; ++t) hmax = fmaxf(hmax, __builtin_fabsf(h[t]));
          } else {
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.h) + idx) =
                make_uint2(f32_to_bf16_bits(h[0]) | (f32_to_bf16_bits(h[1]) << 16),
                           f32_to_bf16_bits(h[2]) | (f32_to_bf16_bits(h[3]) << 16));
          }
        }
      }
    }
    if (T == DT_E4M3) {
      hmax = wave_max(hmax);
      if (lane == 0 && hmax > 0.0f) atomicMax(a.hmax_bits, __float_as_uint(hmax));
    }
  } else {
    float scale = 1.0f;
    if (T == DT_E4M3) scale = (*a.sh) * a.w2_scale[e];
#pragma unroll
    for (int j = 0; j < kPfTB; ++j) {
      const int pos = mb * kPfTok + 64 * wc + 16 * j + r16;
      const int f = a.sorted_ids[pos];
      if (f < a.P) {
        const float m = scale * a.topk_w[f];
#pragma unroll
        for (int i = 0; i < kPfTA; ++i) {
          float* dst = a.y + (size_t)pos * a.K + nt * kPfRows + 128 * wr + 16 * i + 4 * g;
          st16(dst, i32x4{__float_as_int(acc[i][j][0] * m), __float_as_int(acc[i][j][1] * m),
                          __float_as_int(acc[i][j][2] * m), __float_as_int(acc[i][j][3] * m)});
        }
      }
    }
  }
}

// The prefill kernels take bf16 x bf16 or E4M3 x E4M3 operands, alignment
// blocks of at least 128 rows, and (down product) a hidden size that is a
// multiple of the 256-row weight tile.
bool pf_applies(const GemmArgs& a, bool gemm1) {
  const bool types = (a.wt == DT_BF16 && (gemm1 ? a.xt == DT_BF16 : true)) ||
                     (a.wt == DT_E4M3 && (gemm1 ? a.xt == DT_E4M3 : true));
  if (!types || a.block_m < kPfTok) return false;
  return gemm1 ? (a.N % 128 == 0) : (a.K % kPfRows == 0);
}

template <int T, bool G1>
static int pf_launch(const GemmArgs& a, hipStream_t st) {
  static bool attr_set = false;  // per process: one device's attribute covers the kernel
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&pf_gemm_kernel<T, G1>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kPfLdsBytes);
    if (err != hipSuccess) return (int)err;
    attr_set = true;
  }
  const int ntiles = G1 ? a.N / 128 : a.K / kPfRows;
  dim3 grid(ntiles, a.max_blocks);  // block_m >= 128: max_blocks counts 128-row tiles
  hipLaunchKernelGGL((pf_gemm_kernel<T, G1>), grid, dim3(kPfThreads), kPfLdsBytes, st, a);
  return (int)hipGetLastError();
}

int launch_gemm1_prefill(const GemmArgs& a, hipStream_t st) {
  return a.wt == DT_E4M3 ? pf_launch<DT_E4M3, true>(a, st) : pf_launch<DT_BF16, true>(a, st);
}
int launch_gemm2_prefill(const GemmArgs& a, hipStream_t st) {
  return a.wt == DT_E4M3 ? pf_launch<DT_E4M3, false>(a, st) : pf_launch<DT_BF16, false>(a, st);
}

}  // namespace moe
