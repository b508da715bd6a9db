// launch.hpp -- host-side launchers of the gfx950 kernels (internal to the
// library; the public interface is include/moe.h).  Each returns 0 or the
// hipError_t of the failed launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

namespace moe {

constexpr int kMaxDevices = 64;

// Thread-safe one-time set-up per device (kernel attributes such as the
// dynamic LDS limit): the first caller on a device runs f, which returns 0 or
// a hipError_t, and every caller on that device gets that result.  Declare one
// function-local static instance per set-up site.
struct OncePerDevice {
  std::once_flag flag[kMaxDevices];
  std::atomic<int> result[kMaxDevices];
  template <class F>
  int run(F&& f) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
      return (int)hipErrorInvalidDevice;
    std::call_once(flag[dev], [&] { result[dev].store(f()); });
    return result[dev].load();
  }
};

constexpr int kMaxPartials = 1024;

// Linear router projection + top-k (route_project.hip); dtype DT_BF16 or
// DT_F32 for both x [M,K] and wr [E,K]; logits may be NULL; ws holds
// route_project_workspace_bytes(M, K, E) bytes of partial sums.
size_t route_project_workspace_bytes(int M, int K, int E);
int launch_route_project(const void* x, const void* wr, int dtype, int M, int K, int E, int k,
                         int renorm, float* logits, int32_t* ids, float* wts, void* ws,
                         hipStream_t st);
int launch_route_topk(const float* logits, int M, int E, int k, int renorm,
                      int32_t* ids, float* wts, hipStream_t stream);

size_t align_workspace_bytes(int M, int topk, int E);
int launch_align(const int32_t* ids, int M, int topk, int E, int bm,
                 int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                 int32_t* pair_pos, int32_t* num_padded, void* ws,
                 hipStream_t stream);

int launch_route_align(const float* logits, int M, int E, int k, int renorm, int bm,
                       int32_t* ids, float* wts, int32_t* sorted_ids, int32_t* block_expert,
                       int32_t* offsets, int32_t* pair_pos, int32_t* num_padded,
                       hipStream_t stream);

int launch_quant_x(const void* x, int xt, size_t n, const float* static_scale,
                   float* partials, uint8_t* xq, float* sx, uint32_t* hmax_bits,
                   hipStream_t stream);
// pre-quantised activations: s_x = *a1_scale into sx, running max of |h| = 0
int launch_fwd_prequant(const float* a1_scale, float* sx, uint32_t* hmax_bits, hipStream_t stream);
// codes of the rows < *num_rows that hold a pair (sorted_ids[row] < P)
int launch_quant_h(const float* h32, int N, int max_rows, const int32_t* num_rows,
                   const int32_t* sorted_ids, int P, const uint32_t* hmax_bits,
                   const float* static_scale, uint8_t* hq, float* sh, hipStream_t stream);

// Rotary embedding + per-head E4M3 quantisation (rope.hip); x [T, nH, D]
// bf16 or f32, D % 16 == 0, nH <= 256; ws holds rope_workspace_bytes().
size_t rope_workspace_bytes(int T, int nH, int D);
int launch_rope_quant(const void* x, int xt, const int32_t* pos, const float* inv_freq, int T,
                      int nH, int D, int interleaved, int inverse, const float* static_scales,
                      uint8_t* codes, float* scales, void* ws, hipStream_t st);

// Arguments of the expert GEMMs (device pointers unless noted).
struct GemmArgs {
  int M, K, N, E, topk, block_m, P;  // host values
  int max_blocks;                    // host upper bound of padded blocks
  int wt, xt, ot;                    // dtype codes (DT_*)
  const void* x;        // activations for GEMM1 (bf16, f32 or E4M3 codes)
  const void* w13;
  const void* w2;
  const float* w13_scale;
  const float* w2_scale;
  const float* sx;       // E4M3 only: scale of x (device scalar)
  const float* sh;       // E4M3 only: scale of h (device scalar)
  const float* topk_w;
  const int32_t* sorted_ids;
  const int32_t* block_expert;
  const int32_t* offsets;
  const int32_t* pair_pos;
  const int32_t* num_padded;
  void* h;               // [cap, N] bf16 (bf16 family) or fp32 (E4M3)
  const void* hq;        // GEMM2 operand: h itself (bf16) or its E4M3 codes
  uint32_t* hmax_bits;   // E4M3: running max |h|
  void* y;               // tile path: [cap, K] expert outputs before the routing
                         // weight, bf16 when the layer output is bf16, else fp32
  void* out;             // [M, K]
  int probe;             // test builds only: gate/up kernels store the scaled
                         // gate and up sums ([cap, 2N] fp32: gate | up) in h
                         // instead of SiLU(gate) * up; the public entry points
                         // always leave it 0
};

#ifdef __HIPCC__
// Probe store of one 4-row MFMA fragment: rows `row` of the [cap, 2N] fp32
// buffer in a.h, gate values at column col, up values at col + N.
__device__ __forceinline__ void probe_store(const GemmArgs& a, size_t row, int col, const float g4[4],
                                            const float u4[4]) {
  float* p = reinterpret_cast<float*>(a.h) + row * 2 * (size_t)a.N + col;
  *reinterpret_cast<float4*>(p) = make_float4(g4[0], g4[1], g4[2], g4[3]);
  *reinterpret_cast<float4*>(p + a.N) = make_float4(u4[0], u4[1], u4[2], u4[3]);
}
#endif

int launch_gemm1_stream(const GemmArgs& a, hipStream_t stream);
bool gemm1_ring_applies(const GemmArgs& a);
int launch_gemm1_ring(const GemmArgs& a, hipStream_t stream);
int launch_gemm2_stream(const GemmArgs& a, hipStream_t stream);
bool gemm2_ring_applies(const GemmArgs& a);
int launch_gemm2_ring(const GemmArgs& a, hipStream_t stream);
bool pf_applies(const GemmArgs& a, bool gemm1);
int launch_gemm1_prefill(const GemmArgs& a, hipStream_t stream);
int launch_gemm2_prefill(const GemmArgs& a, hipStream_t stream);
bool pfq_applies(const GemmArgs& a, bool gemm1);
int launch_gemm1_pfq(const GemmArgs& a, hipStream_t stream);
int launch_gemm2_pfq(const GemmArgs& a, hipStream_t stream);
int launch_gemm1_tile(const GemmArgs& a, hipStream_t stream);
int launch_gemm2_tile(const GemmArgs& a, hipStream_t stream);
int launch_combine(const GemmArgs& a, hipStream_t stream);

// Single-launch decode forward (fused.hip): E4M3 weights, a.x the bf16 or
// fp32 activations, a.h fp32 h, a.hq its codes, a.y per-pair rows, xq the
// codes of x, sync the zero-initialised synchronisation words
// (fused_sync_bytes()).
size_t fused_sync_bytes();
bool fused_decode_applies(const GemmArgs& a);
int launch_fused_decode(const GemmArgs& a, uint8_t* xq, uint32_t* sync, const float* a1_scale,
                        const float* a2_scale, hipStream_t stream);
int launch_cast_bf16(const float* src, uint16_t* dst, size_t n, hipStream_t stream);

// Compute units of the current device (queried once per device).
int device_cu_count();

// Largest M served by the streaming (decode) kernels.
constexpr int kStreamMaxM = 64;

}  // namespace moe
