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

// MFMA instructions per chunk and wave.
template <int T>
constexpr int kPfMfma() {
  return kPfTA * kPfTB * (T == DT_E4M3 ? 1 : 2);
}
constexpr int kPfDs = 2 * (kPfTA + kPfTB);  // fragment reads per chunk and wave

// Scheduling of one chunk's instruction stream: the kPfNI DMA instructions of
// chunk c + 3 and the kPfDs fragment reads of chunk c + 1 are spread over the
// first three quarters of chunk c's MFMAs (a few MFMAs, one read, one DMA
// instruction, ...), so that they issue in the MFMAs' shadow and the reads
// have completed by the next barrier.  sched_group_barrier masks: 0x008 MFMA,
// 0x100 DS read, 0x020 VMEM read.
template <int NMF, int I = 0>
__device__ __forceinline__ void pf_interleave() {
  constexpr int per = (NMF * 3 / 4) / kPfDs;  // MFMAs before each read
  if constexpr (I < kPfDs) {
    __builtin_amdgcn_sched_group_barrier(0x008, per, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if constexpr (I < kPfNI) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    pf_interleave<NMF, I + 1>();
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, NMF - per * kPfDs, 0);
  }
}

// Scheduling of one bf16 half chunk: its NMF MFMAs with the kPfDs / 2
// fragment reads of the next half spread over the first three quarters, and
// (second half) the kPfNI DMA instructions of the refill as well.
template <int NMF, bool DMA, int I = 0>
__device__ __forceinline__ void pf_interleave_half() {
  constexpr int nds = kPfDs / 2;
  constexpr int per = (NMF * 3 / 4) / nds;
  if constexpr (I < nds) {
    __builtin_amdgcn_sched_group_barrier(0x008, per, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if constexpr (DMA && I < kPfNI) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    pf_interleave_half<NMF, DMA, I + 1>();
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, NMF - per * nds, 0);
  }
}

// Raw buffer resource over [base, base + bytes) (gfx9 word 3: 32-bit data).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
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

// Epilogue of a 256 x 128 tile held as 8 x 4 accumulator tiles per wave
// (wave wr, wc of the 2 x 2 grid).  G1: scale, SiLU(gate) * up, h (bf16, or
// fp32 plus the running amax for E4M3).  G2: scale * W2 h -> y.
template <int T, bool G1>
__device__ __forceinline__ void pf_epilogue(const GemmArgs& a, const f32x4 (&acc)[kPfTA][kPfTB],
                                            const int (&fe)[kPfTB], int e, int nt, int mb, int wr,
                                            int wc, int lane) {
  const int r16 = lane & 15, g = lane >> 4;
  if constexpr (G1) {
    float scale = 1.0f;
    if (T == DT_E4M3) scale = (*a.sx) * a.w13_scale[e];
    float hmax = 0.0f;
#pragma unroll
    for (int j = 0; j < kPfTB; ++j) {
      const int pos = mb * kPfTok + 64 * wc + 16 * j + r16;
      if (fe[j] < a.P) {
#pragma unroll
        for (int i = 0; i < kPfTA / 2; ++i) {
          float h[4], g4[4], u4[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            g4[t] = acc[i][j][t] * scale;
            u4[t] = acc[i + kPfTA / 2][j][t] * scale;
            h[t] = silu(g4[t]) * u4[t];
          }
          const int col = nt * 128 + 64 * wr + 16 * i + 4 * g;
          const size_t idx = (size_t)pos * a.N + col;
          if (a.probe) {
            probe_store(a, (size_t)pos, col, g4, u4);
          } else if (T == DT_E4M3) {
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
    // y rows hold W2 h of each pair; the routing weight is applied where the
    // top-k rows of a token are summed.
    float scale = 1.0f;
    if (T == DT_E4M3) scale = (*a.sh) * a.w2_scale[e];
    const bool ybf = a.ot == DT_BF16;
#pragma unroll
    for (int j = 0; j < kPfTB; ++j) {
      const int pos = mb * kPfTok + 64 * wc + 16 * j + r16;
      if (fe[j] < a.P) {
#pragma unroll
        for (int i = 0; i < kPfTA; ++i) {
          const size_t idx = (size_t)pos * a.K + nt * kPfRows + 128 * wr + 16 * i + 4 * g;
          const float v[4] = {acc[i][j][0] * scale, acc[i][j][1] * scale, acc[i][j][2] * scale,
                              acc[i][j][3] * scale};
          if (ybf)
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.y) + idx) =
                make_uint2(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                           f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
          else
            st16(reinterpret_cast<float*>(a.y) + idx,
                 i32x4{__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]), __float_as_int(v[3])});
        }
      }
    }
  }
}

// G1 = true: gate/up product + SiLU * up -> h.  G1 = false: down product
// -> y (one row per sorted position, routing weight not yet applied).
template <int T, bool G1>
__global__ __launch_bounds__(kPfThreads) void pf_gemm_kernel(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int nt, mb;
  pf_task(nt, mb);
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r16 = lane & 15, g = lane >> 4;
  const int wr = wv >> 1, wc = wv & 1;
  const int Kd = G1 ? a.K : a.N;  // contraction length
  constexpr int EB = Family<T>::kBytes;
  const uint32_t rowb = (uint32_t)Kd * EB;
  const int nchunks = (int)(rowb / kPfChunk);
  const int lrow = lane >> 3, pcol = lane & 7;

  // Metadata, all loads in flight together (every index below is inside the
  // arrays for any block below max_blocks, valid or not).
  const int npad = *a.num_padded;
  const int e = a.block_expert[(mb * kPfTok) / a.block_m];
  int fx[kPfXInstr];  // pair index of the token rows this lane's DMA gathers
#pragma unroll
  for (int q = 0; q < kPfXInstr; ++q) fx[q] = a.sorted_ids[mb * kPfTok + 8 * (wv * kPfXInstr + q) + lrow];
  int fe[kPfTB];  // pair index of the token columns this lane's results belong to
#pragma unroll
  for (int j = 0; j < kPfTB; ++j) fe[j] = a.sorted_ids[mb * kPfTok + 64 * wc + 16 * j + r16];
  if (mb * kPfTok >= npad) return;  // uniform: past the last block

  // DMA sources.  A wave's 8 weight instructions cover 64 consecutive tile
  // rows = 64 consecutive rows of one weight matrix (the gate or up block for
  // the gate/up product); the rotation only depends on the row mod 8, so one
  // lane offset serves all of them and the instruction / chunk offsets are
  // scalar.
  __amdgpu_buffer_rsrc_t wres, xres;
  uint32_t w_sbase, x_sbase = 0;
  const uint32_t w_voff = lrow * rowb + pf_logical(lrow, pcol) * 16;
  uint32_t x_voff[kPfXInstr];
  {
    const int r0 = 64 * wv;  // first tile row of this wave's weight DMA
    if (G1) {
      const int h0 = nt * 128 + 64 * (r0 >> 7);  // first intermediate column
      wres = pf_rsrc(reinterpret_cast<const char*>(a.w13) + (size_t)e * 2 * a.N * rowb, 2 * a.N * rowb);
      w_sbase = (uint32_t)((r0 & 127) < 64 ? h0 : a.N + h0) * rowb;
      xres = pf_rsrc(a.x, (uint32_t)a.M * rowb);
#pragma unroll
      for (int q = 0; q < kPfXInstr; ++q) {
        const int r = 8 * (wv * kPfXInstr + q) + lrow;
        const int f = fx[q] < a.P ? fx[q] : 0;  // padding row: any valid row, never stored
        x_voff[q] = (uint32_t)(f / a.topk) * rowb + pf_logical(r, pcol) * 16;
      }
    } else {
      wres = pf_rsrc(reinterpret_cast<const char*>(a.w2) + (size_t)e * a.K * rowb, a.K * rowb);
      w_sbase = (uint32_t)(nt * kPfRows + r0) * rowb;
      xres = pf_rsrc(reinterpret_cast<const char*>(a.hq) + (size_t)mb * kPfTok * rowb, kPfTok * rowb);
      x_sbase = (uint32_t)(32 * wv) * rowb;
#pragma unroll
      for (int q = 0; q < kPfXInstr; ++q) x_voff[q] = lrow * rowb + pf_logical(lrow, pcol) * 16;
    }
  }
  const __amdgpu_buffer_rsrc_t null_res = pf_rsrc(a.x, 0);  // every access out of range

  // DMA of `chunk` into stage `slot`; past the last chunk the instructions
  // still issue (the instruction stream of every chunk is the same) through a
  // resource of size 0, which fetches nothing.
  auto issue = [&](int chunk, int slot) {
    const bool real = chunk < nchunks;
    const __amdgpu_buffer_rsrc_t wr_ = real ? wres : null_res;
    const __amdgpu_buffer_rsrc_t xr_ = real ? xres : null_res;
    char* sb = lds + slot * kPfStageBytes;
    const uint32_t off = (uint32_t)chunk * kPfChunk;
#pragma unroll
    for (int q = 0; q < kPfWInstr; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr_, (__attribute__((address_space(3))) void*)(sb + (wv * kPfWInstr + q) * 1024), 16, w_voff,
          w_sbase + (uint32_t)(8 * q) * rowb + off, 0, kPfAux);
#pragma unroll
    for (int q = 0; q < kPfXInstr; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr_, (__attribute__((address_space(3))) void*)(sb + kPfWBytes + (wv * kPfXInstr + q) * 1024),
          16, x_voff[q], x_sbase + (uint32_t)(8 * q) * (G1 ? 0u : rowb) + off, 0, kPfAux);
  };

  // The empty asm makes each zero accumulator an opaque value of its own:
  // otherwise the compiler shares one zero register among all of them in the
  // first iteration and then shuffles accumulators between registers inside
  // the loop.
  f32x4 acc[kPfTA][kPfTB];
#pragma unroll
  for (int i = 0; i < kPfTA; ++i)
#pragma unroll
    for (int j = 0; j < kPfTB; ++j) {
      acc[i][j] = f32x4{0, 0, 0, 0};
      asm volatile("" : "+a"(acc[i][j]));
    }

  // LDS offsets of this lane's fragments (logical columns g and g + 4); tile
  // i adds i * 16 rows = i * 2048 bytes (the rotation repeats every 8 rows)
  int aoff[2], boff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    aoff[h] = pf_off(128 * wr + r16, g + 4 * h);
    boff[h] = kPfWBytes + pf_off(64 * wc + r16, g + 4 * h);
  }

  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  pf_wait_vmcnt<2 * kPfNI>();
  pf_barrier();

  if constexpr (T == DT_BF16) {
    // bf16: a chunk is two K halves of 32 (16-byte columns g and g + 4 of
    // each row); half 0 of chunk c is in registers when iteration c starts.
    //   multiply half 0 while reading half 1 of chunk c;
    //   wait for chunk c + 1, barrier (every wave holds all of chunk c, so
    //   stage c % 3 is free), refill it with chunk c + 3;
    //   multiply half 1 while reading half 0 of chunk c + 1.
    // Each register set keeps one role, so the loop body is straight-line
    // code; the last iteration reads a stale stage and the DMA past the end
    // fetches nothing, so every iteration is the same.
    i32x4 A0[kPfTA], B0[kPfTB], A1[kPfTA], B1[kPfTB];
    auto load_half = [&](int h, int slot, i32x4 (&A)[kPfTA], i32x4 (&B)[kPfTB]) {
      const char* sb = lds + slot * kPfStageBytes;
#pragma unroll
      for (int j = 0; j < kPfTB; ++j) B[j] = ld16(sb + boff[h] + j * 16 * kPfChunk);
#pragma unroll
      for (int i = 0; i < kPfTA; ++i) A[i] = ld16(sb + aoff[h] + i * 16 * kPfChunk);
    };
    auto mult_half = [&](const i32x4 (&A)[kPfTA], const i32x4 (&B)[kPfTB]) {
#pragma unroll
      for (int i = 0; i < kPfTA; ++i)
#pragma unroll
        for (int j = 0; j < kPfTB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[i]), as_bf16x8(B[j]), acc[i][j],
                                                              0, 0, 0);
    };
    load_half(0, 0, A0, B0);
    for (int c = 0; c < nchunks; ++c) {
      const int slot = c % 3;
      load_half(1, slot, A1, B1);
      mult_half(A0, B0);
      pf_interleave_half<kPfTA * kPfTB, false>();
      pf_wait_vmcnt<kPfNI>();
      pf_barrier();
      issue(c + 3, slot);
      load_half(0, slot == 2 ? 0 : slot + 1, A0, B0);
      mult_half(A1, B1);
      pf_interleave_half<kPfTA * kPfTB, true>();
    }
  } else {
    // E4M3: one MFMA takes a whole 128-byte chunk, so whole chunks are
    // double-buffered: fragments of chunk c are read right after the barrier
    // that publishes it and multiplied one iteration later.
    Raw<T> A0[kPfTA], B0[kPfTB], A1[kPfTA], B1[kPfTB];
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
      for (int i = 0; i < kPfTA; ++i)
#pragma unroll
        for (int j = 0; j < kPfTB; ++j) acc[i][j] = mma(to_op<T>(A[i]), to_op<T>(B[j]), acc[i][j]);
    };
    // Iteration c: wait for chunk c + 1, barrier (chunk c + 1 visible; every
    // wave holds chunk c's fragments, so stage c % 3 is free), refill that
    // stage with chunk c + 3, read chunk c + 1's fragments, multiply chunk c.
    auto step = [&](int c, Raw<T> (&Ac)[kPfTA], Raw<T> (&Bc)[kPfTB], Raw<T> (&An)[kPfTA],
                    Raw<T> (&Bn)[kPfTB]) {
      pf_wait_vmcnt<kPfNI>();
      pf_barrier();
      issue(c + 3, c % 3);
      load_frags((c + 1) % 3, An, Bn);
      compute(Ac, Bc);
      pf_interleave<kPfMfma<T>()>();
    };
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
  }
  pf_wait_vmcnt<0>();  // no DMA may land after the workgroup's LDS is released

  pf_epilogue<T, G1>(a, acc, fe, e, nt, mb, wr, wc, lane);
}

// The prefill kernels take bf16 x bf16 or E4M3 x E4M3 operands, alignment
// blocks of at least 128 rows, and (down product) a hidden size that is a
// multiple of the 256-row weight tile.
bool pf_applies(const GemmArgs& a, bool gemm1) {
  const bool types = (a.wt == DT_BF16 && (gemm1 ? a.xt == DT_BF16 : true)) ||
                     (a.wt == DT_E4M3 && (gemm1 ? a.xt == DT_E4M3 : true));
  if (!types || a.block_m < kPfTok) return false;
  // buffer resources take 32-bit byte ranges
  const size_t wb = (a.wt == DT_E4M3) ? 1 : 2;
  const size_t lim = (size_t)1 << 31;
  if ((size_t)2 * a.N * a.K * wb >= lim || (size_t)a.M * a.K * wb >= lim) return false;
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
