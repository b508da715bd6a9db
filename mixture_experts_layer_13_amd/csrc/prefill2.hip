// prefill2.hip -- expert GEMMs for large token counts: 256 x 256 macro tiles,
// 128 x 128 (four waves) or 64 x 128 (eight waves) per wave.
//
// Same grouped problem as the other expert GEMMs ("Amazon SageMaker AI 上的
// Mixture-of-Experts 内核工程优化", introduction: tokens bucketed per expert,
// one GEMM per expert), computed as Bᵀ·Aᵀ with the weight rows on the MFMA
// row operand.  A workgroup computes 256 weight rows x 256 token rows (one
// 256-row alignment block of one expert); its waves form an (NW / 2) x 2
// grid and each owns (512 / NW) x 128 of the tile as 32 x 32 blocks
// (v_mfma 32x32x16 bf16 or 32x32x64 E4M3).
//
// Why this shape on MI355X (measured): the direct-to-LDS loads of a CU
// sustain about 60 bytes per clock when every wave instruction reads whole
// 128-byte lines (8 rows x 128 bytes), half that with 64-byte row pieces.
// A 256 x 256 tile needs 32 bytes per clock at the full matrix rate (64 KiB
// per 128 bytes of K, 2048 MFMA cycles per SIMD), half of that budget;
// 256 x 128 needs 48.
//
// Operands reach LDS through a two-stage ring; a stage holds 128 bytes of K
// of all 512 rows (64 KiB).  Row r's 16-byte column c sits at physical
// column (c + (r >> 1)) mod 8, which makes the fragment reads of a 32x32 MFMA
// (lane l reads row l mod 32) conflict-free (measured on MI355X).  A chunk
// is consumed in two halves of 64 bytes: half 0's fragments are read while
// the previous chunk's half 1 is multiplied and vice versa, so one register
// set per half suffices.  The refill of a stage starts right after the
// barrier that follows the reads of its second half, and must land one full
// chunk later: there is one barrier per chunk.
//
// The tile order is persistent: one workgroup per CU walks a contiguous
// range of tiles of its XCD, and the ring runs on across tile boundaries.
// The per-tile metadata (pair indices of the token rows, expert of the
// block) and the E4M3 scales come in through the same direct-to-LDS loads,
// so no load returns into registers inside the loop: the compiler has
// nothing to wait for, and the only waits on the memory counter are the
// ring's own.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQRows = 256;                          // weight rows per tile
constexpr int kQTok = 256;                           // token rows per tile
constexpr int kQChunk = 128;                         // bytes of K per row and stage
constexpr int kQWBytes = kQRows * kQChunk;           // 32 KiB
constexpr int kQStage = (kQRows + kQTok) * kQChunk;  // 64 KiB
constexpr int kQMetaBytes = (kQTok + 64) * 4;        // pair ids of the token rows, block expert

// Layout of a workgroup of NW waves: NW / 2 along the weight rows, 2 along
// the token rows.
template <int NW>
struct QL {
  static constexpr int WR = NW / 2;
  static constexpr int WaveRows = kQRows / WR;   // weight rows of one wave
  static constexpr int TA = WaveRows / 32;       // 32-row weight blocks per wave
  static constexpr int Instr = kQRows / 8 / NW;  // ring loads per wave and operand (8 rows each)
  static constexpr int ND = 2 * (TA + 4);        // fragment reads per half
};

__device__ __forceinline__ int q_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int N>
__device__ __forceinline__ void q_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Barrier that first lets this wave's LDS reads complete (no wave refills a
// stage another wave is still reading).
__device__ __forceinline__ void q_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Raw buffer resource over [base, base + bytes): bytes = 0 fetches nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t q_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void q_dma16(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void q_dma4(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 4, voff, 0, 0, 0);
}

// Logical 16-byte column whose data lands at physical column p of LDS row r.
__device__ __forceinline__ int q_logical(int r, int p) { return (p - (r >> 1)) & 7; }

// One tile: coordinates and expert (wave-uniform), and the per-lane source
// offsets of this wave's token-row loads.  valid = 0: past the workgroup's
// range (its loads fetch nothing).
template <int NW>
struct QTile {
  int nt, mb, e, valid;
  uint32_t xv[QL<NW>::Instr];
};

// The lane's index, recomputed at the point of use: a per-lane value kept
// live across the whole tile loop for one use per tile is what the register
// allocator spills first (and a reload from scratch memory waits for every
// load and store in flight).
__device__ __forceinline__ int q_lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Metadata of token block mb into an LDS slot: 256 pair ids, then the
// expert of the block (and 63 entries that are not used).
template <int NW>
__device__ __forceinline__ void q_meta_issue(const GemmArgs& a, char* slot, int mb, int valid, int wv) {
  const int lane = q_lane_here();
  if (wv < 4) {
    const auto ids = q_rsrc(a.sorted_ids + (size_t)mb * kQTok, valid ? kQTok * 4 : 0);
    q_dma4(ids, slot + wv * 256, ((uint32_t)lane + 64u * wv) * 4);
  }
  if (wv == NW - 1) {
    const auto be = q_rsrc(a.block_expert + (size_t)mb * kQTok / a.block_m, valid ? 4 : 0);
    q_dma4(be, slot + kQTok * 4, (uint32_t)lane * 4);
  }
}

// E4M3 scales into LDS (once per workgroup): the E per-expert weight scales
// of the product (E <= 1024), then the activation scale.
template <int T, bool G1, int NW>
__device__ __forceinline__ void q_scales_issue(const GemmArgs& a, char* dst, int wv, int lane) {
  if constexpr (T == DT_E4M3) {
    const auto ws = q_rsrc(G1 ? a.w13_scale : a.w2_scale, (uint32_t)a.E * 4);
    for (int q = wv; q < (a.E + 63) / 64; q += NW) q_dma4(ws, dst + q * 256, (uint32_t)(q * 64 + lane) * 4);
    if (wv == 0) q_dma4(q_rsrc(G1 ? a.sx : a.sh, 4), dst + 1024 * 4, (uint32_t)lane * 4);
  }
}

// A tile's expert (its metadata has landed and a barrier has passed since).
__device__ __forceinline__ void q_tile_head(const GemmArgs& a, int& e_out, const char* slot) {
  const int* ids = reinterpret_cast<const int*>(slot);
  int e = q_uniform(ids[kQTok]);
  e_out = e < 0 ? 0 : (e >= a.E ? a.E - 1 : e);  // slots of invalid tiles hold no expert
}

// A tile's token-row load offsets: load q of wave wv covers tile rows
// 8 (Instr wv + q) .. + 7, lane l row l / 8, physical column l mod 8.
template <bool G1, int NW>
__device__ __forceinline__ void q_tile_xv(const GemmArgs& a, QTile<NW>& t, const char* slot, uint32_t rowb,
                                          int wv, int lane) {
  using L = QL<NW>;
  const int* ids = reinterpret_cast<const int*>(slot);
#pragma unroll
  for (int q = 0; q < L::Instr; ++q) {
    const int r = (wv * L::Instr + q) * 8 + (lane >> 3);  // token row of the tile
    const int lc = q_logical(kQRows + r, lane & 7);
    // padding rows (past the end of the expert's pairs) take an offset past
    // every operand buffer (all under 2 GiB): their loads return zeros and
    // touch no memory, and their products are never stored
    const int f = ids[r];
    const bool real = f >= 0 && f < a.P;
    const uint32_t row = G1 ? (uint32_t)(f / a.topk) * rowb : (uint32_t)r * rowb;
    t.xv[q] = real ? row + lc * 16 : 0x80000000u;
  }
}

// The ring loads of one chunk of tile t into a stage: buffer resources and
// scalar offsets (wave-uniform).  Weight load q of wave wv covers tile rows
// 8 (Instr wv + q) .. + 7; for the gate/up product the rows of wave row wr
// are WaveRows / 2 gate rows, then the up rows of the same intermediate
// columns 128 nt + (WaveRows / 2) wr + ...
template <int NW>
struct QDma {
  __amdgpu_buffer_rsrc_t wres, xres;
  uint32_t wsoff[QL<NW>::Instr];
  const uint32_t* xv;
  uint32_t coff;
  char* dst;
};

template <bool G1, int NW>
__device__ __forceinline__ QDma<NW> q_plan(const GemmArgs& a, const QTile<NW>& t, int chunk, char* stage,
                                           uint32_t rowb, int wv) {
  using L = QL<NW>;
  QDma<NW> d;
  d.coff = (uint32_t)chunk * kQChunk;
  d.dst = stage;
  d.xv = t.xv;
  if (G1) {
    d.wres = q_rsrc(reinterpret_cast<const char*>(a.w13) + (size_t)t.e * 2 * a.N * rowb,
                    t.valid ? 2u * a.N * rowb : 0u);
    d.xres = q_rsrc(a.x, t.valid ? (uint32_t)a.M * rowb : 0u);
  } else {
    d.wres = q_rsrc(reinterpret_cast<const char*>(a.w2) + (size_t)t.e * a.K * rowb,
                    t.valid ? (uint32_t)a.K * rowb : 0u);
    d.xres = q_rsrc(reinterpret_cast<const char*>(a.hq) + (size_t)t.mb * kQTok * rowb,
                    t.valid ? (uint32_t)kQTok * rowb : 0u);
  }
#pragma unroll
  for (int q = 0; q < L::Instr; ++q) {
    const int r0 = (wv * L::Instr + q) * 8;
    int grow;
    if (G1) {
      constexpr int half = L::WaveRows / 2;
      const int wr = r0 / L::WaveRows, within = r0 % L::WaveRows;
      const int col0 = t.nt * 128 + half * wr;
      grow = within < half ? col0 + within : a.N + col0 + within - half;
    } else {
      grow = t.nt * kQRows + r0;
    }
    d.wsoff[q] = (uint32_t)grow * rowb;
  }
  return d;
}

// Load V of a wave's ring loads (weight rows first, then token rows).  The
// rotation of load q's rows depends on q's parity only (its first row is
// 8 (Instr wv + q) and Instr is even).
template <int NW, int V>
__device__ __forceinline__ void q_dma_one(const QDma<NW>& d, const uint32_t (&wvoff)[2], int wv) {
  constexpr int I = QL<NW>::Instr;
  if constexpr (V < I)
    q_dma16(d.wres, d.dst + (wv * I + V) * 1024, wvoff[V & 1], d.wsoff[V] + d.coff);
  else
    q_dma16(d.xres, d.dst + kQWBytes + (wv * I + (V - I)) * 1024, d.xv[V - I], d.coff);
}

template <int NW, int V0, int V1>
__device__ __forceinline__ void q_dmas(const QDma<NW>& d, const uint32_t (&wvoff)[2], int wv) {
  if constexpr (V0 < V1) {
    q_dma_one<NW, V0>(d, wvoff, wv);
    q_dmas<NW, V0 + 1, V1>(d, wvoff, wv);
  }
}

// Fragments of one half chunk (64 bytes of K).  Lane half h = lane / 32 of
// K step k (0, 1) reads logical column 4 H + 2 k + h of half H.  bf16: two
// MFMA K steps of 16 values.  E4M3: one K step of 64, a lane's 32 bytes being
// its K step 0 and 1 columns.
template <int T, int NW>
struct QFrag;
template <int NW>
struct QFrag<DT_BF16, NW> {
  i32x4 a[2][QL<NW>::TA], b[2][4];
};
template <int NW>
struct QFrag<DT_E4M3, NW> {
  i32x8 a[QL<NW>::TA], b[4];
};

// Fragment read D of a half: K step D / (TA + 4) (E4M3: register half),
// token blocks then weight blocks.
template <int T, int NW, int D>
__device__ __forceinline__ void q_read_one(QFrag<T, NW>& F, const char* stage, int aoff, int boff,
                                           const int (&koff)[2]) {
  constexpr int n = QL<NW>::TA + 4, k = D / n, r = D % n;
  if constexpr (T == DT_BF16) {
    if constexpr (r < 4)
      F.b[k][r] = ld16(stage + boff + r * 4096 + koff[k]);
    else
      F.a[k][r - 4] = ld16(stage + aoff + (r - 4) * 4096 + koff[k]);
  } else {
    if constexpr (r < 4) {
      if constexpr (k == 0)
        F.b[r].lo = ld16(stage + boff + r * 4096 + koff[0]);
      else
        F.b[r].hi = ld16(stage + boff + r * 4096 + koff[1]);
    } else {
      if constexpr (k == 0)
        F.a[r - 4].lo = ld16(stage + aoff + (r - 4) * 4096 + koff[0]);
      else
        F.a[r - 4].hi = ld16(stage + aoff + (r - 4) * 4096 + koff[1]);
    }
  }
}

template <int T, int NW, int D0, int D1>
__device__ __forceinline__ void q_reads(QFrag<T, NW>& F, const char* stage, int aoff, int boff,
                                        const int (&koff)[2]) {
  if constexpr (D0 < D1) {
    q_read_one<T, NW, D0>(F, stage, aoff, boff, koff);
    q_reads<T, NW, D0 + 1, D1>(F, stage, aoff, boff, koff);
  }
}

// MFMA K of a half: bf16 K step K / (4 TA), block (K / 4 mod TA, K mod 4);
// E4M3 block (K / 4, K mod 4).  Z: the half is a tile's first, and its first
// K step takes a zero accumulator operand (the MFMA's inline constant 0), so
// that no register holds zeros for the next tile while the loop runs.
template <int T, int NW, int K, bool Z>
__device__ __forceinline__ void q_mma_one(f32x16 (&acc)[QL<NW>::TA][4], const QFrag<T, NW>& F) {
  constexpr int TA = QL<NW>::TA;
  if constexpr (T == DT_BF16) {
    constexpr int s = K / (4 * TA), i = (K / 4) % TA, j = K % 4;
    const f32x16 c = (Z && s == 0) ? f32x16{} : acc[i][j];
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(F.a[s][i]), as_bf16x8(F.b[s][j]), c, 0, 0, 0);
  } else {
    constexpr int i = K / 4, j = K % 4;
    const f32x16 c = Z ? f32x16{} : acc[i][j];
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.a[i], F.b[j], c, 0, 0, 0, 0, 0, 0);
  }
}

// The instruction stream of a half, in a fixed order: MFMA K, then the
// fragment reads of the next half spread over the first three quarters of
// the MFMAs and (DMA) the ring loads evenly over all of them: the loads of
// a CU's waves then arrive at about the rate its vector memory unit takes
// them (bunched up, they stall the issuing wave and with it its MFMAs).
template <int T, int NW, bool DMA, bool READ, bool Z = false, int K = 0>
__device__ __forceinline__ void q_half(f32x16 (&acc)[QL<NW>::TA][4], const QFrag<T, NW>& Fc, QFrag<T, NW>& Fn,
                                       const char* rstage, int aoff, int boff, const int (&koff)[2],
                                       const QDma<NW>& d, const uint32_t (&wvoff)[2], int wv) {
  using L = QL<NW>;
  constexpr int NM = (T == DT_BF16 ? 2 : 1) * L::TA * 4;
  constexpr int NI = 2 * L::Instr;
  if constexpr (K < NM) {
    q_mma_one<T, NW, K, Z>(acc, Fc);
    constexpr int span = NM * 3 / 4;
    constexpr int d0 = K < span ? K * L::ND / span : L::ND, d1 = K < span ? (K + 1) * L::ND / span : L::ND;
    if constexpr (READ) q_reads<T, NW, d0, d1>(Fn, rstage, aoff, boff, koff);
    if constexpr (DMA) {
      constexpr int v0 = K * NI / NM, v1 = (K + 1) * NI / NM;
      q_dmas<NW, v0, v1>(d, wvoff, wv);
    }
    __builtin_amdgcn_sched_barrier(0);
    q_half<T, NW, DMA, READ, Z, K + 1>(acc, Fc, Fn, rstage, aoff, boff, koff, d, wvoff, wv);
  }
}

// One chunk c (in stage ST): multiply half 0 (F0) while reading half 1 of
// the same stage into F1; wait for chunk c + 1, barrier (every wave is done
// with stage ST), refill stage ST with the chunk two ahead (chunk src_chunk
// of tile src); multiply half 1 (F1) while reading half 0 of chunk c + 1
// into F0 (LAST: not here; the last chunk of a tile leaves that read until
// after the epilogue, so that the epilogue has the fragment registers).
template <int T, bool G1, int NW, int ST, bool LAST = false, bool Z = false>
__device__ __forceinline__ void q_step(const GemmArgs& a, f32x16 (&acc)[QL<NW>::TA][4], QFrag<T, NW>& F0,
                                       QFrag<T, NW>& F1, const QTile<NW>& src, int src_chunk, char* stage0,
                                       char* stage1, uint32_t rowb, const uint32_t (&wvoff)[2], int wv, int aoff,
                                       int boff, const int (&koff)[2][2]) {
  char* cur = ST ? stage1 : stage0;
  char* next = ST ? stage0 : stage1;
  const QDma<NW> none{};
  q_half<T, NW, false, true, Z>(acc, F0, F1, cur, aoff, boff, koff[1], none, wvoff, wv);
  q_wait_vmcnt<0>();
  q_barrier();
  const QDma<NW> d = q_plan<G1, NW>(a, src, src_chunk, cur, rowb, wv);
  q_half<T, NW, true, !LAST>(acc, F1, F0, next, aoff, boff, koff[0], d, wvoff, wv);
}

// Epilogue of a wave's (32 TA) x 128 result: acc[i][j] register r holds
// weight row 32 i + 8 (r / 4) + 4 h + r % 4 (h = lane / 32) of the wave and
// token column 32 j + lane % 32.  G1: scale, SiLU(gate) * up -> h (bf16, or
// fp32 plus the running amax for E4M3); gate blocks i < TA / 2, up blocks
// i + TA / 2.  G2: scale * (W2 h) -> y.
template <int T, bool G1, int NW, bool PROBE>
__device__ __forceinline__ void q_epilogue(const GemmArgs& a, const f32x16 (&acc)[QL<NW>::TA][4],
                                           const char* slot, const float* scales, const QTile<NW>& t, int wr,
                                           int wc, int lane) {
  using L = QL<NW>;
  const int r32 = lane & 31, hh = lane >> 5;
  const int* ids = reinterpret_cast<const int*>(slot);
  int fe[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) fe[j] = ids[128 * wc + 32 * j + r32];
  if constexpr (G1) {
    float scale = 1.0f;
    if (T == DT_E4M3) scale = scales[1024] * scales[t.e];
    float hmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = t.mb * kQTok + 128 * wc + 32 * j + r32;
      if (fe[j] >= 0 && fe[j] < a.P) {
#pragma unroll
        for (int i = 0; i < L::TA / 2; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float h[4], g4[4], u4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              g4[r] = acc[i][j][4 * q + r] * scale;
              u4[r] = acc[i + L::TA / 2][j][4 * q + r] * scale;
              h[r] = silu(g4[r]) * u4[r];
            }
            const int col = t.nt * 128 + (L::WaveRows / 2) * wr + 32 * i + 8 * q + 4 * hh;
            const size_t idx = (size_t)pos * a.N + col;
            if constexpr (PROBE) {
              probe_store(a, (size_t)pos, col, g4, u4);
            } else if constexpr (T == DT_E4M3) {
              st16(reinterpret_cast<float*>(a.h) + idx,
                   i32x4{__float_as_int(h[0]), __float_as_int(h[1]), __float_as_int(h[2]), __float_as_int(h[3])});
#pragma unroll
              for (int r = 0; r < 4; ++r) hmax = fmaxf(hmax, __builtin_fabsf(h[r]));
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
    if (T == DT_E4M3) scale = scales[1024] * scales[t.e];
    const bool ybf = a.ot == DT_BF16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = t.mb * kQTok + 128 * wc + 32 * j + r32;
      if (fe[j] >= 0 && fe[j] < a.P) {
#pragma unroll
        for (int i = 0; i < L::TA; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const size_t idx =
                (size_t)pos * a.K + t.nt * kQRows + L::WaveRows * wr + 32 * i + 8 * q + 4 * hh;
            const float v[4] = {acc[i][j][4 * q] * scale, acc[i][j][4 * q + 1] * scale,
                                acc[i][j][4 * q + 2] * scale, acc[i][j][4 * q + 3] * scale};
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

// Epilogue through LDS (four-wave layout, bf16 output): the wave's result is
// written to memory in rounds of 32 token rows x 128 bytes (two 32-column
// blocks).  Each lane first puts its MFMA results (4 consecutive rows of one
// token) into a 4 KiB staging area of the wave, then reads back 16
// contiguous bytes of a token row, so that every store instruction writes 8
// whole 128-byte row segments instead of 32 scattered 8-byte pieces (which
// the write path handles one piece at a time).  Staging row t holds 16-byte
// column c at c ^ (t mod 8).  val(ii, q, r) gives value r of rows 8 q + 4 h
// of block ii of the round; out0 points at element (first token of the
// round, first column of the round) of the output, row stride `stride`
// elements.
//
// The staging accesses are written in assembly.  The compiler cannot tell
// the staging area from the ring stages that the direct-to-LDS loads fill,
// and before any LDS access it cannot place among those loads it waits for
// every load in flight -- here the next tile's first ring loads and, at the
// next tile's start, this epilogue's stores.  The staging area is the
// wave's own and no load targets it; LDS operations of one wave complete in
// order, so the reads see the writes, and the reads wait for themselves in
// the same statement.
__device__ __forceinline__ uint32_t q_lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

template <typename V>
__device__ __forceinline__ void q_stage_round(char* stg, const int* ids, int tok0, int P, char* out0,
                                              size_t stride, int lane, V val) {
  const int r32 = lane & 31, hh = lane >> 5;
  const uint32_t sbase = q_lds_addr(stg);
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = val(ii, q, r);
      const int b = (32 * ii + 8 * q + 4 * hh) * 2;
      const uint32_t dst = sbase + r32 * 128 + ((((b >> 4) ^ (r32 & 7))) << 4) + (b & 15);
      const u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      asm volatile("ds_write_b64 %0, %1" ::"v"(dst), "v"(pk) : "memory");
    }
  const int c = lane & 7;
  uint32_t src[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int t = (lane >> 3) + 8 * rr;
    src[rr] = sbase + t * 128 + ((c ^ (t & 7)) << 4);
  }
  i32x4 d[4];
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3])
      : "v"(src[0]), "v"(src[1]), "v"(src[2]), "v"(src[3])
      : "memory");
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int t = (lane >> 3) + 8 * rr;
    const int f = ids[tok0 + t];
    if (f >= 0 && f < P) st16(out0 + ((size_t)t * stride) * 2 + c * 16, d[rr]);
  }
  // one round at a time: keeps the scheduler from hoisting the accumulator
  // reads of later rounds (which would need more registers than there are)
  __builtin_amdgcn_sched_barrier(0);
}

// Gate/up epilogue through LDS (four-wave layout, bf16 h): SiLU(gate) * up of
// the wave's 64 intermediate columns x 128 token rows, one round of two
// 32-column blocks per 32 token rows (gate blocks i < TA / 2, up blocks
// i + TA / 2).  The stores from registers would write 8-byte pieces of 32
// rows per instruction; the fp32 h of the E4M3 path already goes out as
// 32-byte row pieces and is stored from registers.
template <int NW>
__device__ __forceinline__ void q_epilogue_g1_staged(const GemmArgs& a, const f32x16 (&acc)[QL<NW>::TA][4],
                                                     const char* slot, const QTile<NW>& t, int wr, int wc,
                                                     int lane, char* stg) {
  using L = QL<NW>;
  static_assert(L::TA == 4, "two gate and two up blocks per wave");
  const int* ids = reinterpret_cast<const int*>(slot);
  const size_t row0 = (size_t)t.mb * kQTok + 128 * wc;  // first token row of the wave
  const int col0 = t.nt * 128 + (L::WaveRows / 2) * wr;  // first h column of the wave
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    char* out0 = reinterpret_cast<char*>(a.h) + ((row0 + 32 * j) * a.N + col0) * 2;
    q_stage_round(stg, ids, 128 * wc + 32 * j, a.P, out0, (size_t)a.N, lane, [&](int ii, int q, int r) {
      return silu(acc[ii][j][4 * q + r]) * acc[ii + L::TA / 2][j][4 * q + r];
    });
  }
}

// Down-product epilogue through LDS (four-wave layout): y (bf16) in rounds
// of 32 token rows x 64 columns.
template <int T, int NW>
__device__ __forceinline__ void q_epilogue_staged(const GemmArgs& a, const f32x16 (&acc)[QL<NW>::TA][4],
                                                  const char* slot, const float* scales, const QTile<NW>& t,
                                                  int wr, int wc, int lane, char* stg) {
  using L = QL<NW>;
  const int* ids = reinterpret_cast<const int*>(slot);
  const size_t row0 = (size_t)t.mb * kQTok + 128 * wc;  // first token row of the wave
  float scale = 1.0f;
  if (T == DT_E4M3) scale = scales[1024] * scales[t.e];
  // y rows hold W2 h of each pair; the routing weight is applied where the
  // top-k rows of a token are summed.
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int ib = 0; ib < L::TA; ib += 2) {
      const int col = t.nt * kQRows + L::WaveRows * wr + 32 * ib;
      char* out0 = reinterpret_cast<char*>(a.y) + ((row0 + 32 * j) * a.K + col) * 2;
      q_stage_round(stg, ids, 128 * wc + 32 * j, a.P, out0, (size_t)a.K, lane,
                       [&](int ii, int q, int r) { return acc[ib + ii][j][4 * q + r] * scale; });
    }
}

// G1 = true: gate/up product + SiLU * up -> h.  G1 = false: down product
// -> y (one row per sorted position, routing weight not yet applied).
// Persistent: the tiles (ntiles weight tiles x num_padded / 256 token
// blocks, token block major: tile = mb * ntiles + nt) are split into 8
// contiguous ranges, one per XCD, and the workgroups of an XCD (the hardware
// deals workgroup ids round-robin over the XCDs) take its tiles round-robin.
// Needs an even number, at least 4, of chunks of 128 bytes of K.
// PROBE: the test-only variant whose gate/up epilogue stores the scaled gate
// and up sums (a.probe set); it keeps that epilogue out of the production
// kernel, whose register budget has no room for two epilogues.
template <int T, bool G1, int NW, bool PROBE>
__global__ __launch_bounds__(NW * 64) void pfq_gemm_kernel(GemmArgs a, int ntiles) {
  using L = QL<NW>;
  // separate arrays, so that the compiler can tell the ring's two stages
  // (and the metadata) apart and sees that the fragment reads of one stage
  // never alias the loads in flight into the other
  __shared__ __attribute__((aligned(16))) char stage0[kQStage];
  __shared__ __attribute__((aligned(16))) char stage1[kQStage];
  __shared__ __attribute__((aligned(16))) char meta[2 * kQMetaBytes];
  __shared__ __attribute__((aligned(16))) float scales[1024 + 64];
  // staged epilogues: the down product's, and the bf16 gate/up product's
  __shared__ __attribute__((aligned(16))) char ystage[NW == 4 && (!G1 || (T == DT_BF16 && !PROBE)) ? 4 : 1][4096];
  const int lane = threadIdx.x & 63;
  const int wv = q_uniform(threadIdx.x >> 6);
  const int wr = wv / 2, wc = wv % 2;
  const int Kd = G1 ? a.K : a.N;
  const uint32_t rowb = (uint32_t)Kd * Family<T>::kBytes;
  const int nchunks = (int)(rowb / kQChunk);

  const int nvalid = q_uniform(*a.num_padded) / kQTok;
  const int total = ntiles * nvalid;
  const int per = total / 8, rem = total % 8, xcd = blockIdx.x % 8;
  int task = xcd * per + min(xcd, rem) + (int)blockIdx.x / 8;
  const int end = xcd * per + min(xcd, rem) + per + (xcd < rem ? 1 : 0);
  const int stride = gridDim.x / 8;
  if (task >= end) return;

  // per-lane constants: fragment offsets (row lane % 32 of a 32-row block,
  // rotation (row >> 1) mod 8) and weight-load offsets (load q: rows
  // 8 q .. 8 q + 7 of its group; the rotation repeats every 16 rows, so even
  // and odd q differ)
  const int r32 = lane & 31, hh = lane >> 5;
  int koff[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int k = 0; k < 2; ++k) koff[h][k] = r32 * kQChunk + (((4 * h + 2 * k + hh) + (r32 >> 1)) & 7) * 16;
  uint32_t wvoff[2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
    wvoff[p] = (uint32_t)(lane >> 3) * rowb + q_logical(8 * p + (lane >> 3), lane & 7) * 16;
  const int aoff = L::WaveRows * wr * kQChunk, boff = kQWBytes + 128 * wc * kQChunk;

  // tile metadata: the first tile's now, the next one's one tile ahead
  QTile<NW> cur, nxt;
  cur.valid = 1;
  cur.mb = task / ntiles;
  cur.nt = task % ntiles;
  q_meta_issue<NW>(a, meta, cur.mb, 1, wv);
  q_scales_issue<T, G1, NW>(a, reinterpret_cast<char*>(scales), wv, lane);
  q_wait_vmcnt<0>();
  q_barrier();
  q_tile_head(a, cur.e, meta);
  q_tile_xv<G1, NW>(a, cur, meta, rowb, wv, lane);
  int slot = 0;  // metadata slot of cur
  {
    const int tn = task + stride;
    nxt.valid = q_uniform(tn < end ? 1 : 0);
    const int tk = tn < end ? tn : task;
    nxt.mb = tk / ntiles;
    nxt.nt = tk % ntiles;
    q_meta_issue<NW>(a, meta + kQMetaBytes, nxt.mb, nxt.valid, wv);
  }

  // every tile's first K step writes its accumulators from a zero operand
  f32x16 acc[L::TA][4];
  QFrag<T, NW> F0, F1;

  // prologue: chunks 0 and 1 of the first tile, half 0 of chunk 0
  {
    const QDma<NW> d0 = q_plan<G1, NW>(a, cur, 0, stage0, rowb, wv);
    q_dmas<NW, 0, 2 * L::Instr>(d0, wvoff, wv);
    // chunk 1's DMA must not be scheduled above chunk 0's: the wait below
    // counts chunk 1 as the only loads still allowed in flight
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const QDma<NW> d1 = q_plan<G1, NW>(a, cur, 1, stage1, rowb, wv);
    q_dmas<NW, 0, 2 * L::Instr>(d1, wvoff, wv);
  }
  q_wait_vmcnt<2 * L::Instr>();  // chunk 0
  q_barrier();
  q_reads<T, NW, 0, L::ND>(F0, stage0, aoff, boff, koff[0]);

  while (true) {
    // step c refills stage c mod 2 with chunk c + 2 (of the next tile past
    // the end of this one); the chunk count is even and at least 4
    q_step<T, G1, NW, 0, false, true>(a, acc, F0, F1, cur, 2, stage0, stage1, rowb, wvoff, wv, aoff, boff, koff);
    q_step<T, G1, NW, 1>(a, acc, F0, F1, cur, 3, stage0, stage1, rowb, wvoff, wv, aoff, boff, koff);
    for (int c = 2; c < nchunks - 2; c += 2) {
      q_step<T, G1, NW, 0>(a, acc, F0, F1, cur, c + 2, stage0, stage1, rowb, wvoff, wv, aoff, boff, koff);
      q_step<T, G1, NW, 1>(a, acc, F0, F1, cur, c + 3, stage0, stage1, rowb, wvoff, wv, aoff, boff, koff);
    }
    // the next tile's metadata was issued before this tile's first step and
    // has landed by that step's wait
    q_tile_head(a, nxt.e, meta + (slot ^ 1) * kQMetaBytes);
    q_tile_xv<G1, NW>(a, nxt, meta + (slot ^ 1) * kQMetaBytes, rowb, wv, lane);
    q_step<T, G1, NW, 0>(a, acc, F0, F1, nxt, 0, stage0, stage1, rowb, wvoff, wv, aoff, boff, koff);
    q_step<T, G1, NW, 1, true>(a, acc, F0, F1, nxt, 1, stage0, stage1, rowb, wvoff, wv, aoff, boff, koff);
    // the epilogues stage through LDS (whole 128-byte row segments per
    // store), except the E4M3 gate/up product's fp32 h and the test-only
    // probe output, which store from registers
    if constexpr (NW == 4 && !G1) {
      q_epilogue_staged<T, NW>(a, acc, meta + slot * kQMetaBytes, scales, cur, wr, wc, lane, ystage[wv]);
    } else if constexpr (NW == 4 && T == DT_BF16 && !PROBE) {
      q_epilogue_g1_staged<NW>(a, acc, meta + slot * kQMetaBytes, cur, wr, wc, lane, ystage[wv]);
    } else {
      q_epilogue<T, G1, NW, PROBE>(a, acc, meta + slot * kQMetaBytes, scales, cur, wr, wc, lane);
    }
    task += stride;
    if (task >= end) break;
    cur = nxt;
    slot ^= 1;
    {
      // every wave is done with the old slot (its epilogue read it) before
      // it is refilled with the metadata of the tile after next
      q_barrier();
      const int tn = task + stride;
      nxt.valid = q_uniform(tn < end ? 1 : 0);
      const int tk = tn < end ? tn : task;
      nxt.mb = tk / ntiles;
      nxt.nt = tk % ntiles;
      q_meta_issue<NW>(a, meta + (slot ^ 1) * kQMetaBytes, nxt.mb, nxt.valid, wv);
    }
    q_reads<T, NW, 0, L::ND>(F0, stage0, aoff, boff, koff[0]);  // half 0 of the tile's chunk 0
  }
  q_wait_vmcnt<0>();  // no load may land after the workgroup's LDS is released
}

// Wave count per operand type and product.
template <int T, bool G1>
constexpr int pfq_waves() {
  return 4;
}

// Applicability: bf16 x bf16 or E4M3 x E4M3 operands, bf16 layer output,
// 256-row alignment blocks, tile-aligned weight rows, an even chunk count of at least 4,
// 32-bit byte ranges for the buffer resources, E <= 1024 (scales staged in
// LDS).
bool pfq_applies(const GemmArgs& a, bool gemm1) {
  const bool types = (a.wt == DT_BF16 && (gemm1 ? a.xt == DT_BF16 : true)) ||
                     (a.wt == DT_E4M3 && (gemm1 ? a.xt == DT_E4M3 : true));
  if (!types || a.block_m % kQTok != 0 || a.E > 1024) return false;
  if (!gemm1 && a.ot != DT_BF16) return false;  // y is staged as bf16
  const size_t eb = a.wt == DT_E4M3 ? 1 : 2;
  const size_t rowb = (size_t)(gemm1 ? a.K : a.N) * eb;
  if (rowb % (2 * kQChunk) != 0 || rowb / kQChunk < 4) return false;
  const size_t lim = (size_t)1 << 31;
  if ((size_t)2 * a.N * a.K * eb >= lim || (size_t)a.M * a.K * eb >= lim) return false;
  return gemm1 ? (a.N % 128 == 0) : (a.K % kQRows == 0);
}

template <int T, bool G1>
static int pfq_launch(const GemmArgs& a, hipStream_t st) {
  constexpr int NW = pfq_waves<T, G1>();
  const int ntiles = G1 ? a.N / 128 : a.K / kQRows;
  const long long blocks = (long long)a.max_blocks * 128 / kQTok;  // max_blocks counts 128-row blocks
  const long long tasks = (long long)ntiles * blocks;
  long long g = tasks < device_cu_count() ? tasks : device_cu_count();
  g = g / 8 * 8;
  if (g < 8) g = 8;
  if (G1 && a.probe)
    hipLaunchKernelGGL((pfq_gemm_kernel<T, G1, NW, true>), dim3((unsigned)g), dim3(NW * 64), 0, st, a, ntiles);
  else
    hipLaunchKernelGGL((pfq_gemm_kernel<T, G1, NW, false>), dim3((unsigned)g), dim3(NW * 64), 0, st, a, ntiles);
  return (int)hipGetLastError();
}

int launch_gemm1_pfq(const GemmArgs& a, hipStream_t st) {
  return a.wt == DT_E4M3 ? pfq_launch<DT_E4M3, true>(a, st) : pfq_launch<DT_BF16, true>(a, st);
}
int launch_gemm2_pfq(const GemmArgs& a, hipStream_t st) {
  return a.wt == DT_E4M3 ? pfq_launch<DT_E4M3, false>(a, st) : pfq_launch<DT_BF16, false>(a, st);
}

}  // namespace moe
