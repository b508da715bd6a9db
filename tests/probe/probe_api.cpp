// probe_api.cpp -- test-only C ABI over the expert GEMM kernels of the fused
// MoE library, built into a separate library (libmoe_probe.so) next to the
// tests; the public library never exports these entry points.
//
// With integer-valued operands every fp32 partial sum of an expert product is
// an exact integer, so the gate and up sums of the gate/up kernels and the
// down kernels' outputs can be compared bit for bit with an integer matrix
// product -- a check of the product (A B)^T = B^T A^T that the kernels compute
// with the weights on the MFMA row operand ("Amazon SageMaker AI 上的
// Mixture-of-Experts 内核工程优化", section "Swap-AB for WGMMA utilization").
// The gate/up kernels run with GemmArgs::probe set, which replaces their
// SiLU(gate) * up epilogue by a store of the two scaled sums.
#include "common.hpp"
#include "launch.hpp"

#include <hip/hip_runtime.h>

namespace {

moe::GemmArgs base_args(int M, int K, int N, int E, int topk, int block_m, int max_blocks) {
  moe::GemmArgs g{};
  g.M = M;
  g.K = K;
  g.N = N;
  g.E = E;
  g.topk = topk;
  g.block_m = block_m;
  g.P = M * topk;
  g.max_blocks = max_blocks;
  return g;
}

}  // namespace

extern "C" {

// Gate/up sums of every routed pair: gu [cap, 2N] fp32 (gate | up) at the
// pair's sorted position.  family 0: the decode kernels (M <= 64), 1: the
// tile kernels.  x: [M, K] in w_dtype's activation type (bf16 for bf16 and
// f32 weights -- f32 x for f32 weights --, E4M3 codes for E4M3 weights).
// Returns 0 or a hipError_t / -1 for an unknown family.
int moe_probe_gate_up(int M, int K, int N, int E, int topk, int block_m, int max_blocks,
                      int w_dtype, const void* x, const void* w13, const float* w13_scale,
                      const float* sx, const int32_t* sorted_ids, const int32_t* block_expert,
                      const int32_t* offsets, const int32_t* num_padded, uint32_t* hmax_bits,
                      float* gu, int family, void* stream) {
  moe::GemmArgs g = base_args(M, K, N, E, topk, block_m, max_blocks);
  g.wt = w_dtype;
  g.xt = (w_dtype == moe::DT_F32 && family == 0) ? moe::DT_F32
         : (w_dtype == moe::DT_E4M3)             ? moe::DT_E4M3
                                                 : moe::DT_BF16;
  g.ot = moe::DT_F32;
  g.x = x;
  g.w13 = w13;
  g.w13_scale = w13_scale;
  g.sx = sx;
  g.sorted_ids = sorted_ids;
  g.block_expert = block_expert;
  g.offsets = offsets;
  g.num_padded = num_padded;
  g.hmax_bits = hmax_bits;
  g.h = gu;
  g.probe = 1;
  hipStream_t st = (hipStream_t)stream;
  if (family == 0) return moe::launch_gemm1_stream(g, st);
  if (family == 1) return moe::launch_gemm1_tile(g, st);
  return -1;
}

// Down product and weighted combine: out [M, K] (out_dtype) from the
// intermediate h [cap, N] (bf16, or E4M3 codes for E4M3 weights) at the
// pairs' sorted positions.  family 0: the decode kernels (the expert ring,
// or for f32 weights the streaming kernel with the combine fused), 1: the
// tile kernels; the ring and the tile kernels write per-pair rows to y
// [cap, K] (out_dtype), then the combine runs.
int moe_probe_down(int M, int K, int N, int E, int topk, int block_m, int max_blocks, int w_dtype,
                   int out_dtype, const void* h, const void* w2, const float* w2_scale,
                   const float* sh, const float* topk_w, const int32_t* sorted_ids,
                   const int32_t* block_expert, const int32_t* offsets, const int32_t* pair_pos,
                   const int32_t* num_padded, void* y, void* out, int family, void* stream) {
  moe::GemmArgs g = base_args(M, K, N, E, topk, block_m, max_blocks);
  g.wt = w_dtype;
  g.xt = (w_dtype == moe::DT_E4M3) ? moe::DT_E4M3 : moe::DT_BF16;
  g.ot = out_dtype;
  g.w2 = w2;
  g.w2_scale = w2_scale;
  g.sh = sh;
  g.hq = h;
  g.topk_w = topk_w;
  g.sorted_ids = sorted_ids;
  g.block_expert = block_expert;
  g.offsets = offsets;
  g.pair_pos = pair_pos;
  g.num_padded = num_padded;
  g.y = y;
  g.out = out;
  hipStream_t st = (hipStream_t)stream;
  if (family == 0 && !moe::gemm2_ring_applies(g)) return moe::launch_gemm2_stream(g, st);
  if (family <= 1) {
    int err = family == 0 ? moe::launch_gemm2_ring(g, st) : moe::launch_gemm2_tile(g, st);
    return err ? err : moe::launch_combine(g, st);
  }
  return -1;
}

}  // extern "C"
