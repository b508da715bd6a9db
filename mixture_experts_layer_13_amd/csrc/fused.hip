// fused.hip -- the decode forward with E4M3 expert weights in one launch:
// activation scale and codes, gate/up with SiLU(gate) * up, the scale and
// codes of h, the down projection and the weighted top-k combine.
//
// The pages' FP8 path pulls the data from HBM once and keeps the per-token
// work on chip in one hardware pass instead of discrete scaling, GEMM and
// aggregation kernels ("Amazon SageMaker AI 上的 Mixture-of-Experts 内核工程优化",
// section "Backend routing for FP8 tensor quantization"; "Amazon SageMaker
// AI 上的 MoE 内核工程优化实践", section "Triton 后端路由").  At decode the
// discrete kernels cost mostly their own dispatch and ramp, so this launch
// runs them as phases of one persistent grid:
//
// (pre-quantised activations, the codes and their scale from
// moe_quantize_act, start at C)
//   A  max |x| over a grid-stride share of x   -> barrier 0 (max reduced);
//      up to kSmallX values every workgroup reduces all of x, no barrier
//   B  E4M3 codes of x, s_x = fl32(amax / 448)  -> barrier 1
//   C  gate/up on the weight ring (ring.hpp), h in fp32, each workgroup's
//      max |h|                                  -> barrier 2 (max reduced)
//   D  E4M3 codes of h, s_h = fl32(hmax / 448)  -> barrier 3
//   E  down on the weight ring, y per pair              -> barrier 4
//   F  the weighted top-k combine, every thread one group of 8 outputs.
//
// Every phase computes what the discrete kernels compute, in the same
// arithmetic, so the output equals moe_fused_forward's wherever both run the
// ring kernels.
//
// Grid barrier.  The grid is two workgroups per CU, all resident at once
// (the host checks the occupancy), so a workgroup may wait for every other.
// Arrivals go to kBarGroups counters (workgroup b to counter b mod
// kBarGroups), so that no more than G / kBarGroups atomics queue on one
// address; the arrival that completes a group counter resets it and counts
// the group on a top counter, and the arrival that completes the top counter
// resets it and publishes the barrier's release word.  The other workgroups
// poll the release word with device-scope loads and a short sleep, bounded:
// after kSpinLimit polls a workgroup records the barrier in the error word
// and goes on (its results are then wrong, but every wave ends).  Release
// words and maxima carry the call's epoch (one more than the last call's),
// so neither needs a reset; the epoch word advances when the call's first
// barrier (0 or 1) completes, when every workgroup has read it.
//
// Hand-offs between phases: every value one workgroup writes for another is
// stored device-coherent (sc1) before the writer arrives at the next barrier
// and is read either device-coherent or on first touch (no L2 of the grid
// has read that line since the launch began: the launch starts with clean
// caches, and the codes are written in 128-byte lines of one writer each).
#include "ring.hpp"

namespace moe {

constexpr int kLineWords = 32;  // 128-byte line
constexpr int kBarGroups = 16;
constexpr int kFusedBarriers = 5;
constexpr int kSpinLimit = 1 << 20;
// sync words: epoch, error, then per barrier kBarGroups group counters, the
// top counter, the 64-bit maximum and kBarGroups copies of the release word
// (each in its own line)
constexpr int kWEpoch = 0;
constexpr int kWErr = kLineWords;
constexpr int kWBar = 2 * kLineWords;
constexpr int kBarLines = 2 * kBarGroups + 2;  // groups, top, max, release copies
constexpr size_t kFusedSyncBytes = (size_t)(kWBar + kFusedBarriers * kBarLines * kLineWords) * 4;
constexpr int kFusedWpc = 2;
constexpr int kSlotBytes = 64;
constexpr size_t kSmallX = 32768;  // values of x every workgroup reduces itself

static_assert(kFusedSyncBytes <= 32768, "sync buffer");
static_assert(kWErr * 4 == 128, "error word offset");

// Synchronisation words are written with atomic read-modify-writes, which
// are performed at the device-coherent level, and read with device-scope
// operations (the compiler turns the idempotent or-0 of rmw_read into a
// device-scope load); every XCD has its own L2, and a plain load could be
// served from a line that L2 holds.
__device__ __forceinline__ uint32_t rmw_read(uint32_t* p) {
  return __hip_atomic_fetch_or(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void rmw_write(uint32_t* p, uint32_t v) {
  (void)__hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid barrier b (all threads of the workgroup call it).  payload >= 0: this
// workgroup's contribution to the barrier's maximum, returned reduced over
// the grid (contributions of 0 are skipped: a maximum whose tag is not this
// call's epoch reads as 0).  first: the call's first barrier (advances the
// epoch).  The maximum is raised on the group's word (next to its counter)
// and the group's last arrival folds it into the barrier's word, so that no
// more than one group's atomics queue on one address.  Each group polls its
// own copy of the release word.
__device__ float grid_barrier(uint32_t* sync, int b, uint32_t epoch, float payload, bool first,
                              float* bcast) {
  // the stores of every wave have completed (device-coherent ones at the
  // device level) before this workgroup is counted
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* bar = sync + kWBar + b * kBarLines * kLineWords;
    uint32_t* top = bar + kBarGroups * kLineWords;
    unsigned long long* mx = reinterpret_cast<unsigned long long*>(top + kLineWords);
    uint32_t* rel = top + 2 * kLineWords;  // kBarGroups copies, one line each
    const unsigned long long tag = (unsigned long long)epoch << 32;
    const int G = gridDim.x;
    const int grp = blockIdx.x % kBarGroups;
    const int ngroups = G < kBarGroups ? G : kBarGroups;
    const uint32_t members = (uint32_t)(G / kBarGroups + (grp < G % kBarGroups ? 1 : 0));
    uint32_t* gc = bar + grp * kLineWords;
    unsigned long long* gmx = reinterpret_cast<unsigned long long*>(gc + 2);
    if (payload > 0.0f) {
      (void)__hip_atomic_fetch_max(gmx, tag | __float_as_uint(payload), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
      wait_vmcnt<0>();
    }
    const uint32_t old = __hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == members - 1u) {
      rmw_write(gc, 0u);
      if (payload >= 0.0f) {
        const unsigned long long m =
            __hip_atomic_fetch_or(gmx, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((m >> 32) == epoch && (uint32_t)m != 0u)
          (void)__hip_atomic_fetch_max(mx, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_vmcnt<0>();
      }
      const uint32_t o2 = __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (o2 == (uint32_t)ngroups - 1u) {
        rmw_write(top, 0u);
        if (first) rmw_write(sync + kWEpoch, epoch);
        wait_vmcnt<0>();
        for (int q = 0; q < ngroups; ++q) rmw_write(rel + q * kLineWords, epoch);
      }
    }
    int it = 0;
    while (rmw_read(rel + grp * kLineWords) != epoch) {
      if (++it > kSpinLimit) {
        __hip_atomic_fetch_or(sync + kWErr, 1u << b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    float r = 0.0f;
    if (payload >= 0.0f) {
      const unsigned long long m =
          __hip_atomic_fetch_or(mx, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      r = (m >> 32) == epoch ? __uint_as_float((uint32_t)m) : 0.0f;
    }
    *bcast = r;
  }
  __syncthreads();
  const float r = *bcast;
  __syncthreads();
  return r;
}

template <int XT>
__device__ __forceinline__ void fused_load8(const void* x, size_t i, float v[8]) {
  if (XT == DT_BF16) {
    const i32x4 q = ld16(reinterpret_cast<const uint16_t*>(x) + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_bits_to_f32((uint32_t)q[j] & 0xffffu);
      v[2 * j + 1] = bf16_bits_to_f32((uint32_t)q[j] >> 16);
    }
  } else {
    const i32x4 a = ld16(reinterpret_cast<const float*>(x) + i);
    const i32x4 b = ld16(reinterpret_cast<const float*>(x) + i + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = __int_as_float(a[j]);
      v[4 + j] = __int_as_float(b[j]);
    }
  }
}

// Eight codes E4M3(fl32(v / s)), packed little-endian (common.hpp
// e4m3_codes4; r = fl32(1 / s)).
__device__ __forceinline__ uint2 codes8(const float v[8], float s, float r, bool fast) {
  return make_uint2(e4m3_codes4(v[0], v[1], v[2], v[3], s, r, fast), e4m3_codes4(v[4], v[5], v[6], v[7], s, r, fast));
}

__device__ __forceinline__ float block_max_ring(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kRingThreads / kWave; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

template <int OT>
__device__ __forceinline__ void fused_combine(const GemmArgs& a, size_t gtid, size_t gthreads) {
  const auto yr = dev_rsrc(a.y);
  constexpr int ES = OT == DT_BF16 ? 2 : 4;
  const size_t rows = (size_t)(*a.num_padded);
  const int groups = a.K / 8;
  const size_t items = (size_t)a.M * groups;
  for (size_t it = gtid; it < items; it += gthreads) {
    const int t = (int)(it / groups), n = (int)(it - (size_t)t * groups) * 8;
    const int rb = n >> 5, c = n & 31;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    for (int j0 = 0; j0 < a.topk; j0 += 8) {
      int pos[8];
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = j0 + j < a.topk;
        pos[j] = ok ? a.pair_pos[(size_t)t * a.topk + j0 + j] : -1;
        w[j] = ok ? a.topk_w[(size_t)t * a.topk + j0 + j] : 0.0f;
      }
      i32x4 q[8][2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t at =
            (uint32_t)((((size_t)rb * rows + (pos[j] < 0 ? 0 : pos[j])) * 32 + c) * ES);
#pragma unroll
        for (int u = 0; u < (OT == DT_BF16 ? 1 : 2); ++u)
          q[j][u] = pos[j] >= 0 ? coh_ld16(yr, at + 16 * u) : i32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (pos[j] < 0) continue;
        if (OT == DT_BF16) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[2 * i] += w[j] * bf16_bits_to_f32((uint32_t)q[j][0][i] & 0xffffu);
            v[2 * i + 1] += w[j] * bf16_bits_to_f32((uint32_t)q[j][0][i] >> 16);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[i] += w[j] * __int_as_float(q[j][0][i]);
            v[4 + i] += w[j] * __int_as_float(q[j][1][i]);
          }
        }
      }
    }
    const size_t o = (size_t)t * a.K + n;
    if (OT == DT_BF16) {
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + o;
      *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      *reinterpret_cast<uint2*>(out + 4) = make_uint2(pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    } else {
      float* out = reinterpret_cast<float*>(a.out) + o;
      st16(out, i32x4{__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]), __float_as_int(v[3])});
      st16(out + 4, i32x4{__float_as_int(v[4]), __float_as_int(v[5]), __float_as_int(v[6]), __float_as_int(v[7])});
    }
  }
}

// One ring phase as ring_gemm_kernel<E4M3, 0, D, ...> runs it: column groups
// of two 16-row blocks where that removes an eighth of the groups.
template <bool G1>
__device__ __forceinline__ void fused_ring(const GemmArgs& a, int GT, char* lds, RingFused fz) {
  if (a.P <= 16) {  // no expert holds two blocks: no pairing scan
    ring_run<DT_E4M3, 1, kRingD, G1, true>(a, GT, lds, nullptr, 0, fz);
    __syncthreads();
    return;
  }
  int base;
  const int npair = pair_scan(a, reinterpret_cast<int*>(lds + kRingD * kG1StageBytes), base);
  const int nb = *a.num_padded / a.block_m;
  if (kPairGain * (nb - npair) >= nb && npair < nb) {
    int* heads = reinterpret_cast<int*>(lds);
    pair_heads(a, base, heads);
    ring_run<DT_E4M3, 2, kRingD - 1, G1, true>(a, GT, lds, heads, npair, fz);
  } else {
    ring_run<DT_E4M3, 1, kRingD, G1, true>(a, GT, lds, nullptr, 0, fz);
  }
  __syncthreads();  // the ring's LDS is free again
}

// Four waves per SIMD (at most 128 VGPRs): two workgroups of five waves
// on a CU need 3 + 3 + 2 + 2 wave slots, but measured on MI355X a second
// workgroup is only placed beside the first when every SIMD can take a
// fourth wave -- at 141 VGPRs (three per SIMD) only one workgroup per CU
// was resident and half the grid waited for the other half to finish.
template <int XT>
__global__ __attribute__((amdgpu_flat_work_group_size(kRingThreads, kRingThreads),
                         amdgpu_waves_per_eu(4, 8)))
void fused_decode_kernel(
    GemmArgs a, uint8_t* xq, uint32_t* sync, int GT1, int GT2, const float* a1_scale,
    const float* a2_scale) {
  // the first kSlotBytes of the dynamic LDS hold the workgroup's reduction
  // and broadcast slots, the ring's LDS follows
  extern __shared__ __attribute__((aligned(16))) char lds_all[];
  float* red = reinterpret_cast<float*>(lds_all);  // kRingThreads / kWave
  float& bcast = red[8];
  float& hmax_slot = red[9];
  uint32_t& epoch_slot = reinterpret_cast<uint32_t*>(lds_all)[10];
  char* lds = lds_all + kSlotBytes;
  const int tid = threadIdx.x;
  const size_t gthreads = (size_t)gridDim.x * kRingThreads;
  const size_t gtid = (size_t)blockIdx.x * kRingThreads + tid;

  if (tid == 0) {
    epoch_slot = rmw_read(sync + kWEpoch) + 1u;
    hmax_slot = 0.0f;
  }
  __syncthreads();
  const uint32_t epoch = epoch_slot;

  // pre-quantised activations (XT = E4M3: the codes with their scale in
  // a1_scale) skip phases A and B
  constexpr bool pre = XT == DT_E4M3;
  float sx = 1.0f;
  if constexpr (pre) {
    sx = *a1_scale;
  } else {
    // ---- A: s_x
    const size_t nx = (size_t)a.M * a.K;  // a multiple of 8
    const bool small_x = nx <= kSmallX;
    if (a1_scale) {
      sx = *a1_scale;
    } else {
      // small x: every workgroup reduces all of it (from L2 after the first
      // touch) and no barrier is needed; else a grid-stride share each
      const size_t i0 = small_x ? (size_t)tid * 8 : gtid * 8;
      const size_t step = small_x ? (size_t)kRingThreads * 8 : gthreads * 8;
      float m = 0.0f;
      for (size_t i = i0; i < nx; i += step) {
        float v[8];
        fused_load8<XT>(a.x, i, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(v[j]));
      }
      m = block_max_ring(m, red);
      const float amax = small_x ? m : grid_barrier(sync, 0, epoch, m, true, &bcast);
      sx = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    }

    // ---- B: codes of x
    {
      const auto xr = dev_rsrc(xq);
      const float rx = 1.0f / sx;
      const bool fx = e4m3_fast_scale(sx, rx);
      for (size_t i = gtid * 8; i < nx; i += gthreads * 8) {
        float v[8];
        fused_load8<XT>(a.x, i, v);
        coh_st8(xr, (uint32_t)i, codes8(v, sx, rx, fx));
      }
    }
    grid_barrier(sync, 1, epoch, -1.0f, a1_scale != nullptr || small_x, &bcast);
  }

  // ---- C: gate/up
  GemmArgs g1 = a;
  g1.x = pre ? a.x : xq;
  g1.xt = DT_E4M3;
  fused_ring<true>(g1, GT1, lds, RingFused{sx, &hmax_slot});

  // ---- s_h
  float sh;
  if (a2_scale) {
    grid_barrier(sync, 2, epoch, -1.0f, pre, &bcast);
    sh = *a2_scale;
  } else {
    const float hm = grid_barrier(sync, 2, epoch, hmax_slot, pre, &bcast);
    sh = (hm == 0.0f) ? 1.0f : hm / 448.0f;
  }

  // ---- D: codes of h ([num_padded, N] fp32, read device-coherent; the
  // padding rows' codes are never used: their columns' sums are dropped)
  {
    const size_t rows = (size_t)(*a.num_padded), nh = rows * a.N;
    const auto hr = dev_rsrc(a.h);
    const auto qr = dev_rsrc(a.hq);
    const float rh = 1.0f / sh;
    const bool fh = e4m3_fast_scale(sh, rh);
    for (size_t i = gtid * 8; i < nh; i += gthreads * 8) {
      const size_t r = i / a.N, n = i - r * a.N;  // 8 columns of one 16-column block
      if (a.sorted_ids[r] >= a.P) continue;
      const uint32_t at = (uint32_t)((((n >> 4) * rows + r) * 16 + (n & 15)) * 4);
      const i32x4 p = coh_ld16(hr, at), q = coh_ld16(hr, at + 16);
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = __int_as_float(p[j]);
        v[4 + j] = __int_as_float(q[j]);
      }
      coh_st8(qr, (uint32_t)i, codes8(v, sh, rh, fh));
    }
  }
  grid_barrier(sync, 3, epoch, -1.0f, false, &bcast);

  // ---- E: down and the combine
  fused_ring<false>(a, GT2, lds, RingFused{sh, nullptr});
  grid_barrier(sync, 4, epoch, -1.0f, false, &bcast);

  // ---- F: out[t, n .. n + 7] = sum over the slots, in slot order, of
  // w[t, j] * y[pair_pos[t, j]] (the combine kernel's arithmetic), y read
  // device-coherent from its tiled layout [K / 32][rows][32]
  if (a.ot == DT_BF16)
    fused_combine<DT_BF16>(a, gtid, gthreads);
  else
    fused_combine<DT_F32>(a, gtid, gthreads);

  if (blockIdx.x == 0 && tid == 0) {
    const_cast<float*>(a.sx)[0] = sx;
    const_cast<float*>(a.sh)[0] = sh;
  }
}

// ------------------------------------------------------------------ launch

size_t fused_sync_bytes() { return kFusedSyncBytes; }

using FusedG1 = RingSize<DT_E4M3, 0, kRingD, kFusedWpc, true>;
using FusedG2 = RingSize<DT_E4M3, 0, kRingD, kFusedWpc, false>;

static size_t fused_lds(const GemmArgs& a) {
  return kSlotBytes + max(FusedG1::lds(a), FusedG2::lds(a));
}

// The launch shape fused_decode_kernel assumes: E4M3 weights, x in bf16 or
// fp32 or already E4M3 codes, 16-row alignment blocks whose pairing scan covers E, rows of whole
// ring stages, every 32-bit byte offset in range, and LDS for two
// workgroups per CU.
bool fused_decode_applies(const GemmArgs& a) {
  if (a.wt != DT_E4M3 || !(a.xt == DT_BF16 || a.xt == DT_F32 || a.xt == DT_E4M3)) return false;
  if (!(a.ot == DT_BF16 || a.ot == DT_F32)) return false;
  if (a.M < 1 || a.M > kStreamMaxM || a.block_m != 16) return false;
  if (a.N % 16 || a.K % 32) return false;
  GemmArgs r = a;
  r.xt = DT_E4M3;
  if (!ring_rows(r, a.K) || !ring_rows(r, a.N) || !ring_pair_fits(r)) return false;
  const long long cap = (long long)a.P + (long long)min(a.E, a.P) * (a.block_m - 1);
  if (cap * a.N * 4 >= (1LL << 32) || cap * a.K * 4 >= (1LL << 32) || (long long)a.M * a.K >= (1LL << 32))
    return false;
  return fused_lds(a) <= (size_t)160 * 1024 / kFusedWpc;
}

template <int XT>
static int fused_setup() {
  // every workgroup of the grid must be resident at once: the dynamic LDS
  // limit is raised to what two workgroups per CU leave, and the occupancy
  // at that size must be two
  static OncePerDevice once;
  return once.run([] {
    const void* k = (const void*)fused_decode_kernel<XT>;
    int err = (int)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       160 * 1024 / kFusedWpc);
    if (err) return err;
    int n = 0;
    err = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kRingThreads,
                                                            160 * 1024 / kFusedWpc);
    if (err) return err;
    return n >= kFusedWpc ? 0 : (int)hipErrorCooperativeLaunchTooLarge;
  });
}

int launch_fused_decode(const GemmArgs& a, uint8_t* xq, uint32_t* sync, const float* a1_scale,
                        const float* a2_scale, hipStream_t st) {
  const int err = a.xt == DT_BF16 ? fused_setup<DT_BF16>()
                  : a.xt == DT_F32 ? fused_setup<DT_F32>() : fused_setup<DT_E4M3>();
  if (err) return err;
  const dim3 grid(kFusedWpc * device_cu_count());
  const size_t lds = fused_lds(a);
  const int gt1 = FusedG1::table_rows(a), gt2 = FusedG2::table_rows(a);
  if (a.xt == DT_BF16)
    hipLaunchKernelGGL(fused_decode_kernel<DT_BF16>, grid, dim3(kRingThreads), lds, st, a, xq, sync,
                       gt1, gt2, a1_scale, a2_scale);
  else if (a.xt == DT_E4M3)
    hipLaunchKernelGGL(fused_decode_kernel<DT_E4M3>, grid, dim3(kRingThreads), lds, st, a, xq, sync,
                       gt1, gt2, a1_scale, a2_scale);
  else
    hipLaunchKernelGGL(fused_decode_kernel<DT_F32>, grid, dim3(kRingThreads), lds, st, a, xq, sync,
                       gt1, gt2, a1_scale, a2_scale);
  return (int)hipGetLastError();
}

}  // namespace moe
