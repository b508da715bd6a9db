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
// Workgroup: WR (weight rows) x 2 (tokens) waves -- 4 x 2 waves of 64 x 64
// (two per SIMD) or 2 x 2 of 128 x 64 (one per SIMD, E4M3 gate/up) -- each
// with its accumulators in the accumulation registers and its operand
// fragments double-buffered in registers.  For the gate/up product a wave's
// rows are gate rows followed by the up rows of the same intermediate
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
// Wave layout of a workgroup: WR waves along the weight rows x 2 along the
// token rows; each wave owns (256 / WR) x 64 of the tile.
template <int WR>
struct PfL {
  static constexpr int WC = 2;
  static constexpr int Waves = WR * WC;
  static constexpr int Threads = Waves * kWave;
  static constexpr int WaveRows = kPfRows / WR;          // weight rows of one wave
  static constexpr int WaveTok = kPfTok / WC;            // token rows of one wave
  static constexpr int WInstr = kPfWBytes / 1024 / Waves;  // DMA instructions per wave and chunk
  static constexpr int XInstr = kPfXBytes / 1024 / Waves;
  static constexpr int WDmaRows = kPfRows / Waves;       // tile rows of one wave's weight DMA
  static constexpr int XDmaRows = kPfTok / Waves;
  static constexpr int TA = WaveRows / 16;               // 16-row weight tiles per wave
  static constexpr int TB = WaveTok / 16;                // 16-row token tiles per wave
  static constexpr int NI = WInstr + XInstr;
  static constexpr int Ds = 2 * (TA + TB);               // fragment reads per chunk and wave
  template <int T>
  static constexpr int mfma() {                          // MFMAs per chunk and wave
    return TA * TB * (T == DT_E4M3 ? 1 : 2);
  }
};

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

// Scheduling of one chunk's instruction stream: the NI DMA instructions of
// chunk c + 3 and the Ds fragment reads of chunk c + 1 are spread over the
// first three quarters of chunk c's MFMAs (a few MFMAs, one read, one DMA
// instruction, ...), so that they issue in the MFMAs' shadow and the reads
// have completed by the next barrier.  sched_group_barrier masks: 0x008 MFMA,
// 0x100 DS read, 0x020 VMEM read.
template <int WR, int NMF, int I = 0>
__device__ __forceinline__ void pf_interleave() {
  using L = PfL<WR>;
  constexpr int per = (NMF * 3 / 4) / L::Ds;  // MFMAs before each read
  if constexpr (I < L::Ds) {
    __builtin_amdgcn_sched_group_barrier(0x008, per, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if constexpr (I < L::NI) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    pf_interleave<WR, NMF, I + 1>();
  } else {
    __builtin_amdgcn_sched_group_barrier(0x008, NMF - per * L::Ds, 0);
  }
}

// Scheduling of one bf16 half chunk: its NMF MFMAs with the Ds / 2 fragment
// reads of the next half spread over the first three quarters, and (second
// half) the NI DMA instructions of the refill as well.
template <int WR, int NMF, bool DMA, int I = 0>
__device__ __forceinline__ void pf_interleave_half() {
  using L = PfL<WR>;
  constexpr int nds = L::Ds / 2;
  constexpr int per = (NMF * 3 / 4) / nds;
  if constexpr (I < nds) {
    __builtin_amdgcn_sched_group_barrier(0x008, per, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if constexpr (DMA && I < L::NI) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    pf_interleave_half<WR, NMF, DMA, I + 1>();
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
template <int T, bool G1, int WR>
__device__ __forceinline__ void pf_epilogue(const GemmArgs& a,
                                            const f32x4 (&acc)[PfL<WR>::TA][PfL<WR>::TB],
                                            const int (&fe)[PfL<WR>::TB], int e, int nt, int mb, int wr,
                                            int wc, int lane) {
  using L = PfL<WR>;
  const int r16 = lane & 15, g = lane >> 4;
  if constexpr (G1) {
    float scale = 1.0f;
    if (T == DT_E4M3) scale = (*a.sx) * a.w13_scale[e];
    float hmax = 0.0f;
#pragma unroll
    for (int j = 0; j < L::TB; ++j) {
      const int pos = mb * kPfTok + L::WaveTok * wc + 16 * j + r16;
      if (fe[j] < a.P) {
#pragma unroll
        for (int i = 0; i < L::TA / 2; ++i) {
          float h[4], g4[4], u4[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            g4[t] = acc[i][j][t] * scale;
            u4[t] = acc[i + L::TA / 2][j][t] * scale;
            h[t] = silu(g4[t]) * u4[t];
          }
          const int col = nt * 128 + (L::WaveRows / 2) * wr + 16 * i + 4 * g;
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
                make_uint2(pack_bf16x2(h[0], h[1]),
                           pack_bf16x2(h[2], h[3]));
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
    for (int j = 0; j < L::TB; ++j) {
      const int pos = mb * kPfTok + L::WaveTok * wc + 16 * j + r16;
      if (fe[j] < a.P) {
#pragma unroll
        for (int i = 0; i < L::TA; ++i) {
          const size_t idx = (size_t)pos * a.K + nt * kPfRows + L::WaveRows * wr + 16 * i + 4 * g;
          const float v[4] = {acc[i][j][0] * scale, acc[i][j][1] * scale, acc[i][j][2] * scale,
                              acc[i][j][3] * scale};
          if (ybf)
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.y) + idx) =
                make_uint2(pack_bf16x2(v[0], v[1]),
                           pack_bf16x2(v[2], v[3]));
          else
            st16(reinterpret_cast<float*>(a.y) + idx,
                 i32x4{__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]), __float_as_int(v[3])});
        }
      }
    }
  }
}

// One tile: its coordinates and expert (wave-uniform; readfirstlane keeps
// them in scalar registers, so that the buffer resources built from them are
// scalar too) and the per-lane DMA row offsets of its token rows and pair
// indices of its result columns.  valid = 0: no such tile (its DMA fetches
// nothing).
template <int WR>
struct PfTile {
  int nt, mb, e, valid;
  uint32_t x_voff[PfL<WR>::XInstr];
  int fe[PfL<WR>::TB];  // pair index of the token columns this lane's results belong to
};

// Tile `task`, in token block major order (mb = task / ntiles, nt = task %
// ntiles: the weight tiles that share one token block are neighbours, which
// measured slightly faster on MI355X than weight tile major); task < 0 gives
// an invalid tile.
template <int T, bool G1, int WR>
__device__ __forceinline__ PfTile<WR> pf_tile(const GemmArgs& a, int task, int ntiles,
                                              uint32_t rowb, int wv, int lane) {
  using L = PfL<WR>;
  PfTile<WR> t;
  t.valid = __builtin_amdgcn_readfirstlane(task >= 0 ? 1 : 0);
  const int tk = __builtin_amdgcn_readfirstlane(task >= 0 ? task : 0);  // in-range metadata; never fetched
  t.mb = tk / ntiles;
  t.nt = tk % ntiles;
  const int lrow = lane >> 3, pcol = lane & 7, r16 = lane & 15, wc = wv % L::WC;
  t.e = __builtin_amdgcn_readfirstlane(a.block_expert[(t.mb * kPfTok) / a.block_m]);
  int fx[L::XInstr];  // pair index of the token rows this lane's DMA gathers
#pragma unroll
  for (int q = 0; q < L::XInstr; ++q) fx[q] = a.sorted_ids[t.mb * kPfTok + 8 * (wv * L::XInstr + q) + lrow];
#pragma unroll
  for (int j = 0; j < L::TB; ++j) t.fe[j] = a.sorted_ids[t.mb * kPfTok + L::WaveTok * wc + 16 * j + r16];
#pragma unroll
  for (int q = 0; q < L::XInstr; ++q) {
    if (G1) {
      const int r = 8 * (wv * L::XInstr + q) + lrow;
      const int f = fx[q] < a.P ? fx[q] : 0;  // padding row: any valid row, never stored
      t.x_voff[q] = (uint32_t)(f / a.topk) * rowb + pf_logical(r, pcol) * 16;
    } else {
      t.x_voff[q] = lrow * rowb + pf_logical(lrow, pcol) * 16;
    }
  }
  return t;
}

// DMA of chunk cc of the current tile (cc >= nchunks: chunk cc - nchunks
// of the next tile) into stage `slot`.  The instructions always issue (the
// instruction stream of every chunk is the same); chunks that do not exist
// go through a resource of size 0, which fetches nothing.  A wave's WInstr
// weight instructions cover WDmaRows consecutive tile rows, which are
// consecutive rows of one weight matrix (for the gate/up product all gate or
// all up rows, as WDmaRows is at most half a wave's rows); the rotation only
// depends on the row mod 8, so one lane offset (w_voff) serves all of them
// and the instruction and chunk offsets are scalar.
template <int T, bool G1, int WR>
__device__ __forceinline__ void pf_issue(const GemmArgs& a, char* lds, const PfTile<WR>& cur,
                                         const PfTile<WR>& nxt, int cc, int slot, int nchunks,
                                         uint32_t rowb, uint32_t w_voff, int wv) {
  using L = PfL<WR>;
  const bool in_cur = cc < nchunks;
  const int chunk = in_cur ? cc : cc - nchunks;
  const bool real = in_cur || (nxt.valid && chunk < nchunks);
  const int e = in_cur ? cur.e : nxt.e, nt = in_cur ? cur.nt : nxt.nt, mb = in_cur ? cur.mb : nxt.mb;
  const int r0 = L::WDmaRows * wv;  // first tile row of this wave's weight DMA
  __amdgpu_buffer_rsrc_t wres, xres;
  uint32_t w_sb, x_sb = 0;
  if (G1) {
    // wave rows: L::WaveRows / 2 gate rows, then the up rows of the same columns
    constexpr int half = L::WaveRows / 2;
    const int within = r0 % L::WaveRows;
    const int h0 = nt * 128 + half * (r0 / L::WaveRows);  // first intermediate column
    wres = pf_rsrc(reinterpret_cast<const char*>(a.w13) + (size_t)e * 2 * a.N * rowb, real ? 2 * a.N * rowb : 0);
    w_sb = (uint32_t)(within < half ? h0 + within : a.N + h0 + within - half) * rowb;
    xres = pf_rsrc(a.x, real ? (uint32_t)a.M * rowb : 0);
  } else {
    wres = pf_rsrc(reinterpret_cast<const char*>(a.w2) + (size_t)e * a.K * rowb, real ? a.K * rowb : 0);
    w_sb = (uint32_t)(nt * kPfRows + r0) * rowb;
    xres = pf_rsrc(reinterpret_cast<const char*>(a.hq) + (size_t)mb * kPfTok * rowb, real ? kPfTok * rowb : 0);
    x_sb = (uint32_t)(L::XDmaRows * wv) * rowb;
  }
  char* sb = lds + slot * kPfStageBytes;
  const uint32_t off = (uint32_t)chunk * kPfChunk;
#pragma unroll
  for (int q = 0; q < L::WInstr; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        wres, (__attribute__((address_space(3))) void*)(sb + (wv * L::WInstr + q) * 1024), 16, w_voff,
        w_sb + (uint32_t)(8 * q) * rowb + off, 0, kPfAux);
#pragma unroll
  for (int q = 0; q < L::XInstr; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        xres, (__attribute__((address_space(3))) void*)(sb + kPfWBytes + (wv * L::XInstr + q) * 1024), 16,
        in_cur ? cur.x_voff[q] : nxt.x_voff[q], x_sb + (uint32_t)(8 * q) * (G1 ? 0u : rowb) + off, 0,
        kPfAux);
}

// G1 = true: gate/up product + SiLU * up -> h.  G1 = false: down product
// -> y (one row per sorted position, routing weight not yet applied).
//
// persist = 1: the grid holds one workgroup per CU (a multiple of 8); the
// valid tiles (ntiles weight tiles x num_padded / 128 token blocks, in
// pf_tile's order) are split into 8 contiguous ranges, one per XCD, and the
// workgroups of an XCD take its tiles round-robin.  The DMA ring runs on
// across tile boundaries: the last three steps of a tile already fetch the
// first chunks of the next one, and the epilogue of a tile overlaps that
// fetch.  Needs nchunks >= 3 (and even for E4M3, whose fragments alternate
// between two register sets per chunk).  persist = 0: one tile per
// workgroup of an (ntiles, max_blocks) grid.
template <int T, bool G1, int WR>
__global__ __launch_bounds__(PfL<WR>::Threads) void pf_gemm_kernel(GemmArgs a, int ntiles, int persist) {
  using L = PfL<WR>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r16 = lane & 15, g = lane >> 4;
  const int wr = wv / L::WC, wc = wv % L::WC;
  const int Kd = G1 ? a.K : a.N;  // contraction length
  constexpr int EB = Family<T>::kBytes;
  const uint32_t rowb = (uint32_t)Kd * EB;
  const int nchunks = (int)(rowb / kPfChunk);
  const int lrow = lane >> 3, pcol = lane & 7;

  const int nvalid = *a.num_padded / kPfTok;
  int task, stride, end;
  if (persist) {
    const int total = ntiles * nvalid;
    const int per = total / 8, rem = total % 8;
    const int xcd = blockIdx.x % 8;
    task = xcd * per + min(xcd, rem) + blockIdx.x / 8;
    end = xcd * per + min(xcd, rem) + per + (xcd < rem ? 1 : 0);
    stride = gridDim.x / 8;
  } else {
    int nt, mb;
    pf_task(nt, mb);
    if (mb >= nvalid) return;  // uniform: past the last block
    task = mb * ntiles + nt;
    end = task + 1;
    stride = 1;
  }
  if (task >= end) return;

  PfTile<WR> cur = pf_tile<T, G1, WR>(a, task, ntiles, rowb, wv, lane);
  PfTile<WR> nxt = pf_tile<T, G1, WR>(a, task + stride < end ? task + stride : -1, ntiles, rowb, wv, lane);
  const uint32_t w_voff = lrow * rowb + pf_logical(lrow, pcol) * 16;

  auto issue = [&](int cc, int slot) {
    pf_issue<T, G1, WR>(a, lds, cur, nxt, cc, slot, nchunks, rowb, w_voff, wv);
  };

  // The empty asm makes each zero accumulator an opaque value of its own:
  // otherwise the compiler shares one zero register among all of them in the
  // first iteration and then shuffles accumulators between registers inside
  // the loop.
  f32x4 acc[L::TA][L::TB];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < L::TA; ++i)
#pragma unroll
      for (int j = 0; j < L::TB; ++j) {
        acc[i][j] = f32x4{0, 0, 0, 0};
        asm volatile("" : "+a"(acc[i][j]));
      }
  };
  zero_acc();

  // LDS offsets of this lane's fragments (logical columns g and g + 4); tile
  // i adds i * 16 rows = i * 2048 bytes (the rotation repeats every 8 rows)
  int aoff[2], boff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    aoff[h] = pf_off(L::WaveRows * wr + r16, g + 4 * h);
    boff[h] = kPfWBytes + pf_off(L::WaveTok * wc + r16, g + 4 * h);
  }

  // chunks 0, 1, 2 in this order (the wait counts chunks 1 and 2 as the
  // loads still allowed in flight), so the scheduler may not interleave them
  issue(0, 0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  issue(1, 1);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  issue(2, 2);
  pf_wait_vmcnt<2 * L::NI>();
  pf_barrier();

  int q0 = 0;  // ring position of the current tile's chunk 0 (mod 3)
  if constexpr (T == DT_BF16) {
    // bf16: a chunk is two K halves of 32 (16-byte columns g and g + 4 of
    // each row); half 0 of chunk c is in registers when step c starts:
    //   multiply half 0 while reading half 1 of chunk c;
    //   wait for chunk c + 1, barrier (every wave holds all of chunk c, so
    //   its stage is free), refill it with chunk c + 3;
    //   multiply half 1 while reading half 0 of chunk c + 1 (of the next tile
    //   after the last chunk).
    // Each register set keeps one role, so the loop body is straight-line.
    i32x4 A0[L::TA], B0[L::TB], A1[L::TA], B1[L::TB];
    auto load_half = [&](int h, int slot, i32x4 (&A)[L::TA], i32x4 (&B)[L::TB]) {
      const char* sb = lds + slot * kPfStageBytes;
#pragma unroll
      for (int j = 0; j < L::TB; ++j) B[j] = ld16(sb + boff[h] + j * 16 * kPfChunk);
#pragma unroll
      for (int i = 0; i < L::TA; ++i) A[i] = ld16(sb + aoff[h] + i * 16 * kPfChunk);
    };
    auto mult_half = [&](const i32x4 (&A)[L::TA], const i32x4 (&B)[L::TB]) {
#pragma unroll
      for (int i = 0; i < L::TA; ++i)
#pragma unroll
        for (int j = 0; j < L::TB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[i]), as_bf16x8(B[j]), acc[i][j],
                                                              0, 0, 0);
    };
    load_half(0, 0, A0, B0);
    while (true) {
      for (int c = 0; c < nchunks; ++c) {
        const int slot = (q0 + c) % 3;
        load_half(1, slot, A1, B1);
        mult_half(A0, B0);
        pf_interleave_half<WR, L::TA * L::TB, false>();
        pf_wait_vmcnt<L::NI>();
        pf_barrier();
        issue(c + 3, slot);
        load_half(0, slot == 2 ? 0 : slot + 1, A0, B0);
        mult_half(A1, B1);
        pf_interleave_half<WR, L::TA * L::TB, true>();
      }
      pf_epilogue<T, G1, WR>(a, acc, cur.fe, cur.e, cur.nt, cur.mb, wr, wc, lane);
      task += stride;
      if (task >= end) break;
      q0 = (q0 + nchunks) % 3;
      cur = nxt;
      nxt = pf_tile<T, G1, WR>(a, task + stride < end ? task + stride : -1, ntiles, rowb, wv, lane);
      zero_acc();
    }
  } else {
    // E4M3: one MFMA takes a whole 128-byte chunk, so whole chunks are
    // double-buffered: fragments of chunk c are read right after the barrier
    // that publishes it and multiplied one step later.
    Raw<T> A0[L::TA], B0[L::TB], A1[L::TA], B1[L::TB];
    auto load_frags = [&](int slot, Raw<T> (&A)[L::TA], Raw<T> (&B)[L::TB]) {
      const char* sb = lds + slot * kPfStageBytes;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int j = 0; j < L::TB; ++j) B[j].q[h] = ld16(sb + boff[h] + j * 16 * kPfChunk);
#pragma unroll
        for (int i = 0; i < L::TA; ++i) A[i].q[h] = ld16(sb + aoff[h] + i * 16 * kPfChunk);
      }
    };
    auto compute = [&](const Raw<T> (&A)[L::TA], const Raw<T> (&B)[L::TB]) {
#pragma unroll
      for (int i = 0; i < L::TA; ++i)
#pragma unroll
        for (int j = 0; j < L::TB; ++j) acc[i][j] = mma(to_op<T>(A[i]), to_op<T>(B[j]), acc[i][j]);
    };
    // Step c: wait for chunk c + 1, barrier (chunk c + 1 visible; every wave
    // holds chunk c's fragments, so its stage is free), refill that stage
    // with chunk c + 3, read chunk c + 1's fragments, multiply chunk c.
    auto step = [&](int c, Raw<T> (&Ac)[L::TA], Raw<T> (&Bc)[L::TB], Raw<T> (&An)[L::TA],
                    Raw<T> (&Bn)[L::TB]) {
      const int slot = (q0 + c) % 3;
      pf_wait_vmcnt<L::NI>();
      pf_barrier();
      issue(c + 3, slot);
      load_frags(slot == 2 ? 0 : slot + 1, An, Bn);
      compute(Ac, Bc);
      pf_interleave<WR, L::template mfma<T>()>();
    };
    load_frags(0, A0, B0);
    while (true) {
      int c = 0;
      for (; c + 1 < nchunks; c += 2) {
        step(c, A0, B0, A1, B1);
        step(c + 1, A1, B1, A0, B0);
      }
      if (c < nchunks) step(c, A0, B0, A1, B1);  // odd count: one tile per workgroup only
      pf_epilogue<T, G1, WR>(a, acc, cur.fe, cur.e, cur.nt, cur.mb, wr, wc, lane);
      task += stride;
      if (task >= end) break;
      q0 = (q0 + nchunks) % 3;
      cur = nxt;
      nxt = pf_tile<T, G1, WR>(a, task + stride < end ? task + stride : -1, ntiles, rowb, wv, lane);
      zero_acc();
    }
  }
  pf_wait_vmcnt<0>();  // no DMA may land after the workgroup's LDS is released
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

// Workgroups of a persistent launch: one per CU (the 144 KiB of LDS admit
// one), but at most a quarter of the tile count (small problems still give
// every workgroup a run of tiles), in multiples of the 8 XCDs; 0 = too few
// tiles for a persistent launch.
static int pf_persistent_grid(long long tiles) {
  const int cus = device_cu_count();
  long long g = tiles / 4 < cus ? tiles / 4 : cus;
  return (int)(g / 8 * 8);
}

// Wave layout per operand type and product (measured on MI355X at T = 4096
// and 8192): 8 waves of 64 x 64 for bf16 and the E4M3 down product, 4 waves of
// 128 x 64 for the E4M3 gate/up product.
template <int T, bool G1>
constexpr int pf_wr() {
  return (T == DT_E4M3 && G1) ? 2 : 4;
}

template <int T, bool G1>
static int pf_launch(const GemmArgs& a, hipStream_t st) {
  constexpr int WR = pf_wr<T, G1>();
  using L = PfL<WR>;
  static OncePerDevice attr;
  const int err = attr.run([] {
    return (int)hipFuncSetAttribute(reinterpret_cast<const void*>(&pf_gemm_kernel<T, G1, WR>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, kPfLdsBytes);
  });
  if (err) return err;
  const int ntiles = G1 ? a.N / 128 : a.K / kPfRows;
  const long long rowb = (long long)(G1 ? a.K : a.N) * Family<T>::kBytes;
  const int nchunks = (int)(rowb / kPfChunk);
  const int persist = nchunks >= 3 && (T != DT_E4M3 || nchunks % 2 == 0);
  const long long tasks = (long long)ntiles * a.max_blocks;  // block_m >= 128: 128-row tiles
  const int pgrid = persist ? pf_persistent_grid(tasks) : 0;
  if (pgrid > 0) {
    hipLaunchKernelGGL((pf_gemm_kernel<T, G1, WR>), dim3(pgrid), dim3(L::Threads), kPfLdsBytes, st, a, ntiles, 1);
  } else {
    dim3 grid(ntiles, a.max_blocks);
    hipLaunchKernelGGL((pf_gemm_kernel<T, G1, WR>), grid, dim3(L::Threads), kPfLdsBytes, st, a, ntiles, 0);
  }
  return (int)hipGetLastError();
}

int launch_gemm1_prefill(const GemmArgs& a, hipStream_t st) {
  return a.wt == DT_E4M3 ? pf_launch<DT_E4M3, true>(a, st) : pf_launch<DT_BF16, true>(a, st);
}
int launch_gemm2_prefill(const GemmArgs& a, hipStream_t st) {
  return a.wt == DT_E4M3 ? pf_launch<DT_E4M3, false>(a, st) : pf_launch<DT_BF16, false>(a, st);
}

}  // namespace moe
