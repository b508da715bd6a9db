// moe_api.cpp -- the C ABI of include/moe.h: host-side validation, workspace
// layout and kernel dispatch.  Validation never touches the GPU; a call that
// returns a non-zero status has enqueued nothing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

moe_status ok() {
  g_err[0] = 0;
  return MOE_OK;
}

moe_status hip_status(int err, const char* what) {
  if (err == 0) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)err));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int dtype_bytes(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }

constexpr long long kMaxPairs = 1LL << 26;

moe_status check_route_dims(int32_t M, int32_t E, int32_t topk) {
  if (M < 0) return fail(MOE_ERR_SHAPE, "M=%d must be >= 0", M);
  if (E < 1 || E > 1024) return fail(MOE_ERR_SHAPE, "E=%d must be in [1, 1024]", E);
  if (topk < 1 || topk > 64 || topk > E)
    return fail(MOE_ERR_SHAPE, "topk=%d must be in [1, min(E, 64)]", topk);
  if ((long long)M * topk > kMaxPairs)
    return fail(MOE_ERR_SHAPE, "M*topk=%lld exceeds %lld", (long long)M * topk, kMaxPairs);
  return MOE_OK;
}

bool valid_block_m(int32_t bm) {
  return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256;
}

// Workspace layout of moe_fused_forward (offsets in bytes, 256-aligned).
struct Layout {
  size_t partials, scalars, xq, xbf, h, hq, y, total;
};

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// s_x and s_h sit right after the amax partials, where the header says
static_assert(((moe::kMaxPartials * sizeof(float) + 255) & ~(size_t)255) ==
                  MOE_WORKSPACE_SCALES_OFFSET,
              "scales offset");

Layout layout_of(const moe_problem& p) {
  Layout L{};
  const long long cap = moe_align_capacity(p.M, p.topk, p.E, p.block_m);
  const bool fp8 = p.w_dtype == MOE_FP8_E4M3;
  const bool stream_path = p.M <= moe::kStreamMaxM;
  size_t o = 0;
  L.partials = o;
  o = up256(o + moe::kMaxPartials * sizeof(float));
  L.scalars = o;  // sx, sh, hmax bits
  o = up256(o + 16);
  L.xq = o;
  if (fp8) o = up256(o + (size_t)p.M * p.K);
  L.xbf = o;
  if (!fp8 && !stream_path && p.a_dtype == MOE_F32) o = up256(o + (size_t)p.M * p.K * 2);
  L.h = o;
  o = up256(o + (size_t)cap * p.N * (fp8 ? 4 : 2));
  L.hq = o;
  if (fp8) o = up256(o + (size_t)cap * p.N);
  L.y = o;  // per-pair down-projection rows in the output dtype (every path but the
            // f32-weight decode kernel)
  o = up256(o + (size_t)cap * p.K * dtype_bytes(p.out_dtype));
  L.total = o;
  return L;
}

moe_status check_problem(const moe_problem* p) {
  if (!p) return fail(MOE_ERR_NULL, "problem is NULL");
  moe_status s = check_route_dims(p->M, p->E, p->topk);
  if (s) return s;
  if (p->K < 128 || p->K > 65536 || p->K % 128)
    return fail(MOE_ERR_SHAPE, "K=%d must be a multiple of 128 in [128, 65536]", p->K);
  if (p->N < 128 || p->N > 65536 || p->N % 128)
    return fail(MOE_ERR_SHAPE, "N=%d must be a multiple of 128 in [128, 65536]", p->N);
  if (!valid_block_m(p->block_m))
    return fail(MOE_ERR_SHAPE, "block_m=%d must be 16, 32, 64, 128 or 256", p->block_m);
  for (int dt : {p->a_dtype, p->w_dtype, p->out_dtype})
    if (dt < MOE_F32 || dt > MOE_FP8_E4M3) return fail(MOE_ERR_DTYPE, "unknown dtype code %d", dt);
  if (p->a_dtype == MOE_FP8_E4M3 && p->w_dtype != MOE_FP8_E4M3)
    return fail(MOE_ERR_UNSUPPORTED, "E4M3 activations need E4M3 weights");
  if (p->out_dtype == MOE_FP8_E4M3) return fail(MOE_ERR_UNSUPPORTED, "output must be f32 or bf16");
  long long cap = moe_align_capacity(p->M, p->topk, p->E, p->block_m);
  if ((long long)cap * p->K > (1LL << 40))
    return fail(MOE_ERR_SHAPE, "padded rows x K too large");
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int32_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_err; }

int64_t moe_align_capacity(int32_t M, int32_t topk, int32_t E, int32_t block_m) {
  if (M < 0 || topk < 1 || E < 1 || block_m < 1) return -1;
  long long P = (long long)M * topk;
  long long act = P < E ? P : E;
  return P + act * (block_m - 1);
}

moe_status moe_workspace_size(const moe_problem* p, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  moe_status s = check_problem(p);
  if (s) return s;
  Layout L = layout_of(*p);
  size_t a = moe::align_workspace_bytes(p->M, p->topk, p->E);
  *bytes = L.total > a ? L.total : a;
  return ok();
}

moe_status moe_route_topk(const float* logits, int32_t M, int32_t E, int32_t topk,
                          int32_t renormalize, int32_t* topk_ids, float* topk_weights,
                          void* stream) {
  moe_status s = check_route_dims(M, E, topk);
  if (s) return s;
  if (M == 0) return ok();
  if (!logits || !topk_ids || !topk_weights)
    return fail(MOE_ERR_NULL, "logits, topk_ids and topk_weights are required");
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
    return fail(MOE_ERR_ALIGN, "route buffers must be 4-byte aligned");
  int err = moe::launch_route_topk(logits, M, E, topk, renormalize ? 1 : 0, topk_ids,
                                   topk_weights, (hipStream_t)stream);
  return hip_status(err, "route_topk launch");
}

static moe_status check_project_dims(int32_t M, int32_t K, int32_t E) {
  moe_status s = check_route_dims(M, E, 1);
  if (s) return s;
  if (K < 128 || K > 65536 || K % 128)
    return fail(MOE_ERR_SHAPE, "K=%d must be a multiple of 128 in [128, 65536]", K);
  return MOE_OK;
}

moe_status moe_route_project_workspace_size(int32_t M, int32_t K, int32_t E, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  moe_status s = check_project_dims(M, K, E);
  if (s) return s;
  *bytes = moe::route_project_workspace_bytes(M, K, E);
  return ok();
}

moe_status moe_route_project_topk(const void* x, int32_t x_dtype, const void* w_router,
                                  int32_t w_dtype, int32_t M, int32_t K, int32_t E,
                                  int32_t topk, int32_t renormalize, float* logits,
                                  int32_t* topk_ids, float* topk_weights, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  moe_status s = check_route_dims(M, E, topk);
  if (s) return s;
  s = check_project_dims(M, K, E);
  if (s) return s;
  if ((x_dtype != MOE_BF16 && x_dtype != MOE_F32) || (w_dtype != MOE_BF16 && w_dtype != MOE_F32))
    return fail(MOE_ERR_DTYPE, "x and router weight must be MOE_BF16 or MOE_F32");
  if (x_dtype != w_dtype)
    return fail(MOE_ERR_UNSUPPORTED, "x_dtype=%d and w_dtype=%d differ", x_dtype, w_dtype);
  if (M == 0) return ok();
  if (!x || !w_router || !topk_ids || !topk_weights || !workspace)
    return fail(MOE_ERR_NULL, "x, w_router, topk_ids, topk_weights and workspace are required");
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(workspace, 16))
    return fail(MOE_ERR_ALIGN, "x, w_router and workspace must be 16-byte aligned");
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
    return fail(MOE_ERR_ALIGN, "route buffers must be 4-byte aligned");
  const size_t need = moe::route_project_workspace_bytes(M, K, E);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  // the MOE_ dtype codes are the kernels' own (0 f32, 1 bf16)
  int err = moe::launch_route_project(x, w_router, x_dtype, M, K, E, topk, renormalize ? 1 : 0,
                                      logits, topk_ids, topk_weights, workspace,
                                      (hipStream_t)stream);
  return hip_status(err, "route_project launch");
}

moe_status moe_align_permute(const int32_t* topk_ids, int32_t M, int32_t topk, int32_t E,
                             int32_t block_m, int32_t* sorted_pair_ids,
                             int32_t* block_expert_ids, int32_t* expert_offsets,
                             int32_t* pair_pos, int32_t* num_padded, void* workspace,
                             size_t workspace_bytes, void* stream) {
  moe_status s = check_route_dims(M, E, topk);
  if (s) return s;
  if (!valid_block_m(block_m))
    return fail(MOE_ERR_SHAPE, "block_m=%d must be 16, 32, 64, 128 or 256", block_m);
  if (!expert_offsets || !num_padded)
    return fail(MOE_ERR_NULL, "expert_offsets and num_padded are required");
  if (M > 0 && (!topk_ids || !sorted_pair_ids || !block_expert_ids || !pair_pos))
    return fail(MOE_ERR_NULL, "topk_ids, sorted_pair_ids, block_expert_ids, pair_pos are required");
  for (const void* q : {(const void*)topk_ids, (const void*)sorted_pair_ids,
                        (const void*)block_expert_ids, (const void*)expert_offsets,
                        (const void*)pair_pos, (const void*)num_padded})
    if (!aligned(q, 4)) return fail(MOE_ERR_ALIGN, "align buffers must be 4-byte aligned");
  size_t need = moe::align_workspace_bytes(M, topk, E);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace_bytes);
  if (workspace && !aligned(workspace, 16))
    return fail(MOE_ERR_ALIGN, "workspace must be 16-byte aligned");
  int err = moe::launch_align(topk_ids, M, topk, E, block_m, sorted_pair_ids, block_expert_ids,
                              expert_offsets, pair_pos, num_padded, workspace,
                              (hipStream_t)stream);
  return hip_status(err, "align launch");
}

moe_status moe_route_align(const float* logits, int32_t M, int32_t E, int32_t topk,
                           int32_t renormalize, int32_t block_m, int32_t* topk_ids,
                           float* topk_weights, int32_t* sorted_pair_ids,
                           int32_t* block_expert_ids, int32_t* expert_offsets,
                           int32_t* pair_pos, int32_t* num_padded, void* workspace,
                           size_t workspace_bytes, void* stream) {
  moe_status s = check_route_dims(M, E, topk);
  if (s) return s;
  // one workgroup routes one token per wave: worth a launch only up to 8 rows
  // (measured: 2 us slower than two launches at 16, 8 at 32, 23 at 64)
  if ((long long)M * topk > 1024 || M > 8 || M == 0) {
    s = moe_route_topk(logits, M, E, topk, renormalize, topk_ids, topk_weights, stream);
    if (s) return s;
    return moe_align_permute(topk_ids, M, topk, E, block_m, sorted_pair_ids, block_expert_ids,
                             expert_offsets, pair_pos, num_padded, workspace, workspace_bytes,
                             stream);
  }
  if (!valid_block_m(block_m))
    return fail(MOE_ERR_SHAPE, "block_m=%d must be 16, 32, 64, 128 or 256", block_m);
  if (!logits || !topk_ids || !topk_weights || !sorted_pair_ids || !block_expert_ids ||
      !expert_offsets || !pair_pos || !num_padded)
    return fail(MOE_ERR_NULL, "a required pointer is NULL");
  for (const void* q : {(const void*)logits, (const void*)topk_ids, (const void*)topk_weights,
                        (const void*)sorted_pair_ids, (const void*)block_expert_ids,
                        (const void*)expert_offsets, (const void*)pair_pos,
                        (const void*)num_padded})
    if (!aligned(q, 4)) return fail(MOE_ERR_ALIGN, "route/align buffers must be 4-byte aligned");
  int err = moe::launch_route_align(logits, M, E, topk, renormalize ? 1 : 0, block_m, topk_ids,
                                    topk_weights, sorted_pair_ids, block_expert_ids,
                                    expert_offsets, pair_pos, num_padded, (hipStream_t)stream);
  return hip_status(err, "route_align launch");
}

}  // extern "C"

namespace {

// Records a timing event on `st`.  Under stream capture the record is added
// to the graph as an event-record node after the stream's current capture
// dependencies (and becomes the new one), so every replay re-records the
// event at that point; otherwise it is an ordinary hipEventRecord.
int record_timing_event(void* ev, hipStream_t st) {
  if (!ev) return 0;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  unsigned long long id = 0;
  hipGraph_t graph = nullptr;
  const hipGraphNode_t* deps = nullptr;
  size_t ndeps = 0;
  hipError_t e = hipStreamGetCaptureInfo_v2(st, &cs, &id, &graph, &deps, &ndeps);
  if (e == hipSuccess) {
    if (cs != hipStreamCaptureStatusActive) {
      e = hipEventRecord((hipEvent_t)ev, st);
    } else {
      hipGraphNode_t node = nullptr;
      e = hipGraphAddEventRecordNode(&node, graph, deps, ndeps, (hipEvent_t)ev);
      if (e == hipSuccess)
        e = hipStreamUpdateCaptureDependencies(st, &node, 1, hipStreamSetCaptureDependencies);
    }
  }
  if (e != hipSuccess) (void)hipGetLastError();  // reported here, not by the next launch
  return (int)e;
}

// moe_fused_forward with optional events around the two GEMM launches.
moe_status fused_forward(const moe_problem* p, const void* a, const void* w13, const void* w2,
                         const float* w13_scale, const float* w2_scale, const float* a1_scale,
                         const float* a2_scale, const float* topk_weights,
                         const int32_t* sorted_pair_ids, const int32_t* block_expert_ids,
                         const int32_t* expert_offsets, const int32_t* pair_pos,
                         const int32_t* num_padded, void* out, void* workspace,
                         size_t workspace_bytes, void* stream, void* const* events,
                         bool persistent = false, void* sync = nullptr, size_t sync_bytes = 0) {
  moe_status s = check_problem(p);
  if (s) return s;
  if (p->M == 0) return ok();
  if (p->a_dtype == MOE_FP8_E4M3 && !a1_scale)
    return fail(MOE_ERR_NULL, "E4M3 activations need their scale in a1_scale");
  if (persistent) {
    if (!sync) return fail(MOE_ERR_NULL, "sync is NULL");
    if (!aligned(sync, 128)) return fail(MOE_ERR_ALIGN, "sync must be 128-byte aligned");
    if (sync_bytes < MOE_FUSED_SYNC_BYTES)
      return fail(MOE_ERR_WORKSPACE, "sync buffer of %d bytes needed, %zu given",
                  (int)MOE_FUSED_SYNC_BYTES, sync_bytes);
  }
  const bool fp8 = p->w_dtype == MOE_FP8_E4M3;
  if (!a || !w13 || !w2 || !topk_weights || !sorted_pair_ids || !block_expert_ids ||
      !expert_offsets || !pair_pos || !num_padded || !out || !workspace)
    return fail(MOE_ERR_NULL, "a required pointer is NULL");
  if (fp8 && (!w13_scale || !w2_scale))
    return fail(MOE_ERR_NULL, "E4M3 weights need w13_scale and w2_scale");
  for (const void* q : {a, w13, w2, (const void*)out, (const void*)workspace})
    if (!aligned(q, 16)) return fail(MOE_ERR_ALIGN, "x, w13, w2, out, workspace must be 16-byte aligned");
  for (const void* q : {(const void*)topk_weights, (const void*)sorted_pair_ids,
                        (const void*)block_expert_ids, (const void*)expert_offsets,
                        (const void*)pair_pos, (const void*)num_padded,
                        (const void*)w13_scale, (const void*)w2_scale,
                        (const void*)a1_scale, (const void*)a2_scale})
    if (!aligned(q, 4)) return fail(MOE_ERR_ALIGN, "index and scale buffers must be 4-byte aligned");
  {
    const char* o0 = (const char*)out;
    const char* o1 = o0 + (size_t)p->M * p->K * dtype_bytes(p->out_dtype);
    const char* a0 = (const char*)a;
    const char* a1 = a0 + (size_t)p->M * p->K * dtype_bytes(p->a_dtype);
    if (o0 < a1 && a0 < o1) return fail(MOE_ERR_SHAPE, "out aliases the input");
  }
  Layout L = layout_of(*p);
  size_t need = L.total;
  size_t na = moe::align_workspace_bytes(p->M, p->topk, p->E);
  if (na > need) need = na;
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace_bytes);

  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const bool stream_path = p->M <= moe::kStreamMaxM;
  const long long cap = moe_align_capacity(p->M, p->topk, p->E, p->block_m);
  const int tbm = p->block_m < 128 ? p->block_m : 128;

  moe::GemmArgs g{};
  g.M = p->M;
  g.K = p->K;
  g.N = p->N;
  g.E = p->E;
  g.topk = p->topk;
  g.block_m = p->block_m;
  g.P = p->M * p->topk;
  g.max_blocks = (int)(cap / tbm > 0 ? cap / tbm : 1);
  g.wt = p->w_dtype;
  g.ot = p->out_dtype;
  g.w13 = w13;
  g.w2 = w2;
  g.w13_scale = w13_scale;
  g.w2_scale = w2_scale;
  float* scal = (float*)(ws + L.scalars);
  g.sx = scal + 0;
  g.sh = scal + 1;
  g.hmax_bits = (uint32_t*)(scal + 2);
  g.topk_w = topk_weights;
  g.sorted_ids = sorted_pair_ids;
  g.block_expert = block_expert_ids;
  g.offsets = expert_offsets;
  g.pair_pos = pair_pos;
  g.num_padded = num_padded;
  g.h = ws + L.h;
  g.y = ws + L.y;
  g.out = out;

  int err = 0;
  if (persistent) {
    g.x = a;
    g.xt = p->a_dtype;
    g.hq = ws + L.hq;
    if (!moe::fused_decode_applies(g))
      return fail(MOE_ERR_UNSUPPORTED,
                  "the one-launch forward needs E4M3 weights, bf16/f32 activations, "
                  "1 <= M <= 64, block_m 16 and per-pair buffers under 4 GiB");
    err = moe::launch_fused_decode(g, (uint8_t*)(ws + L.xq), (uint32_t*)sync, a1_scale, a2_scale,
                                   st);
    if (err) return hip_status(err, "one-launch forward");
    return ok();
  }
  if (fp8 && p->a_dtype == MOE_FP8_E4M3) {
    // codes made beforehand (moe_quantize_act), their scale in a1_scale
    err = moe::launch_fwd_prequant(a1_scale, scal + 0, g.hmax_bits, st);
    if (err) return hip_status(err, "pre-quantised activation launch");
    g.x = a;
    g.xt = MOE_FP8_E4M3;
  } else if (fp8) {
    err = moe::launch_quant_x(a, p->a_dtype, (size_t)p->M * p->K, a1_scale,
                              (float*)(ws + L.partials), (uint8_t*)(ws + L.xq), scal + 0,
                              g.hmax_bits, st);
    if (err) return hip_status(err, "activation quantisation launch");
    g.x = ws + L.xq;
    g.xt = MOE_FP8_E4M3;
  } else if (!stream_path && p->a_dtype == MOE_F32) {
    err = moe::launch_cast_bf16((const float*)a, (uint16_t*)(ws + L.xbf), (size_t)p->M * p->K, st);
    if (err) return hip_status(err, "activation cast launch");
    g.x = ws + L.xbf;
    g.xt = MOE_BF16;
  } else {
    g.x = a;
    g.xt = p->a_dtype;
  }

  void* prof[4];
  for (int i = 0; i < 4; ++i) prof[i] = events ? events[i] : nullptr;
  if ((err = record_timing_event(prof[0], st))) return hip_status(err, "timing event record");
  err = stream_path ? moe::launch_gemm1_stream(g, st) : moe::launch_gemm1_tile(g, st);
  if (err) return hip_status(err, "gate/up GEMM launch");
  if ((err = record_timing_event(prof[1], st))) return hip_status(err, "timing event record");

  if (fp8) {
    err = moe::launch_quant_h((const float*)g.h, p->N, (int)cap, num_padded, sorted_pair_ids, g.P,
                              g.hmax_bits,
                              a2_scale, (uint8_t*)(ws + L.hq), scal + 1, st);
    if (err) return hip_status(err, "intermediate quantisation launch");
    g.hq = ws + L.hq;
  } else {
    g.hq = g.h;
  }

  if ((err = record_timing_event(prof[2], st))) return hip_status(err, "timing event record");
  if (stream_path && !moe::gemm2_ring_applies(g)) {
    err = moe::launch_gemm2_stream(g, st);  // f32 weights: combine fused
    if (err) return hip_status(err, "down GEMM launch");
  } else {
    err = stream_path ? moe::launch_gemm2_ring(g, st) : moe::launch_gemm2_tile(g, st);
    if (err) return hip_status(err, "down GEMM launch");
    if ((err = record_timing_event(prof[3], st))) return hip_status(err, "timing event record");
    prof[3] = nullptr;
    err = moe::launch_combine(g, st);
    if (err) return hip_status(err, "combine launch");
  }
  if ((err = record_timing_event(prof[3], st))) return hip_status(err, "timing event record");
  return ok();
}

// Workspace of moe_fused_forward_noalloc: one array per device, kept for the
// life of the process.  Its name is a host-side stand-in for the device
// address; host code uses only the address that hipGetSymbolAddress returns
// for the current device.
constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_scratch_once[moe::kMaxDevices];
void* g_scratch_ptr[moe::kMaxDevices];
int g_scratch_err[moe::kMaxDevices];

// Device address of this device's scratch array (looked up once per device,
// with that device current); 0 or a hipError_t.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= moe::kMaxDevices)
    return (int)hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = (int)hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = ptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace

extern "C" {

moe_status moe_fused_forward(const moe_problem* p, const void* a, const void* w13,
                             const void* w2, const float* w13_scale, const float* w2_scale,
                             const float* a1_scale, const float* a2_scale,
                             const float* topk_weights, const int32_t* sorted_pair_ids,
                             const int32_t* block_expert_ids, const int32_t* expert_offsets,
                             const int32_t* pair_pos, const int32_t* num_padded, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return fused_forward(p, a, w13, w2, w13_scale, w2_scale, a1_scale, a2_scale, topk_weights,
                       sorted_pair_ids, block_expert_ids, expert_offsets, pair_pos, num_padded,
                       out, workspace, workspace_bytes, stream, nullptr);
}

moe_status moe_fused_forward_noalloc(
    const moe_problem* p, const void* a, const void* w13, const void* w2,
    const float* w13_scale, const float* w2_scale, const float* a1_scale, const float* a2_scale,
    const float* topk_weights, const int32_t* sorted_pair_ids, const int32_t* block_expert_ids,
    const int32_t* expert_offsets, const int32_t* pair_pos, const int32_t* num_padded, void* out,
    void* stream) {
  moe_status s = check_problem(p);
  if (s) return s;
  size_t need = 0;
  s = moe_workspace_size(p, &need);
  if (s) return s;
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "problem needs %zu bytes of workspace; moe_fused_forward_noalloc holds at most %zu "
                "(use moe_fused_forward with a caller workspace)",
                need, kScratchBytes);
  if (p->M == 0) return ok();
  void* ws = nullptr;
  int err = scratch_address(&ws);
  if (err) return hip_status(err, "scratch address lookup");
  return fused_forward(p, a, w13, w2, w13_scale, w2_scale, a1_scale, a2_scale, topk_weights,
                       sorted_pair_ids, block_expert_ids, expert_offsets, pair_pos, num_padded,
                       out, ws, kScratchBytes, stream, nullptr);
}

moe_status moe_fused_forward_profiled(
    const moe_problem* p, const void* a, const void* w13, const void* w2,
    const float* w13_scale, const float* w2_scale, const float* a1_scale, const float* a2_scale,
    const float* topk_weights, const int32_t* sorted_pair_ids, const int32_t* block_expert_ids,
    const int32_t* expert_offsets, const int32_t* pair_pos, const int32_t* num_padded, void* out,
    void* workspace, size_t workspace_bytes, void* stream, void* const events[4]) {
  return fused_forward(p, a, w13, w2, w13_scale, w2_scale, a1_scale, a2_scale, topk_weights,
                       sorted_pair_ids, block_expert_ids, expert_offsets, pair_pos, num_padded,
                       out, workspace, workspace_bytes, stream, events);
}

moe_status moe_fused_forward_persistent(
    const moe_problem* p, const void* a, const void* w13, const void* w2,
    const float* w13_scale, const float* w2_scale, const float* a1_scale, const float* a2_scale,
    const float* topk_weights, const int32_t* sorted_pair_ids, const int32_t* block_expert_ids,
    const int32_t* expert_offsets, const int32_t* pair_pos, const int32_t* num_padded, void* out,
    void* workspace, size_t workspace_bytes, void* sync, size_t sync_bytes, void* stream) {
  static_assert(MOE_FUSED_SYNC_ERROR_OFFSET == 128, "error word offset");
  if (moe::fused_sync_bytes() > MOE_FUSED_SYNC_BYTES) return fail(MOE_ERR_UNSUPPORTED, "sync size");
  return fused_forward(p, a, w13, w2, w13_scale, w2_scale, a1_scale, a2_scale, topk_weights,
                       sorted_pair_ids, block_expert_ids, expert_offsets, pair_pos, num_padded,
                       out, workspace, workspace_bytes, stream, nullptr, true, sync, sync_bytes);
}

static moe_status check_rope_dims(int32_t T, int32_t n_heads, int32_t head_dim) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T=%d must be >= 0", T);
  if (n_heads < 1 || n_heads > 256) return fail(MOE_ERR_SHAPE, "n_heads=%d must be in [1, 256]", n_heads);
  if (head_dim < 16 || head_dim > 512 || head_dim % 16)
    return fail(MOE_ERR_SHAPE, "head_dim=%d must be a multiple of 16 in [16, 512]", head_dim);
  if ((long long)T * n_heads * head_dim > (1LL << 34))
    return fail(MOE_ERR_SHAPE, "T*n_heads*head_dim too large");
  return MOE_OK;
}

moe_status moe_rope_workspace_size(int32_t T, int32_t n_heads, int32_t head_dim, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_NULL, "bytes is NULL");
  moe_status s = check_rope_dims(T, n_heads, head_dim);
  if (s) return s;
  *bytes = moe::rope_workspace_bytes(T, n_heads, head_dim);
  return ok();
}

moe_status moe_rope_quantize_per_head(const void* x, int32_t x_dtype, const int32_t* positions,
                                      const float* inv_freq, int32_t T, int32_t n_heads,
                                      int32_t head_dim, int32_t interleaved, int32_t inverse,
                                      const float* static_scales, uint8_t* codes, float* scales,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  moe_status s = check_rope_dims(T, n_heads, head_dim);
  if (s) return s;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16)
    return fail(MOE_ERR_DTYPE, "x_dtype must be MOE_F32 or MOE_BF16");
  if (T == 0) return ok();
  if (!x || !positions || !inv_freq || !codes || !scales || !workspace)
    return fail(MOE_ERR_NULL, "x, positions, inv_freq, codes, scales and workspace are required");
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(workspace, 16))
    return fail(MOE_ERR_ALIGN, "x, codes and workspace must be 16-byte aligned");
  if (!aligned(positions, 4) || !aligned(inv_freq, 4) || !aligned(scales, 4) ||
      !aligned(static_scales, 4))
    return fail(MOE_ERR_ALIGN, "positions, inv_freq and scales must be 4-byte aligned");
  const size_t need = moe::rope_workspace_bytes(T, n_heads, head_dim);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  int err = moe::launch_rope_quant(x, x_dtype, positions, inv_freq, T, n_heads, head_dim,
                                   interleaved ? 1 : 0, inverse ? 1 : 0, static_scales, codes,
                                   scales, workspace, (hipStream_t)stream);
  return hip_status(err, "rope launch");
}

moe_status moe_quantize_act(const void* x, int32_t x_dtype, int64_t n, const float* static_scale,
                            uint8_t* codes, float* scale, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16)
    return fail(MOE_ERR_DTYPE, "x_dtype must be MOE_F32 or MOE_BF16");
  if (n < 0 || n % 128) return fail(MOE_ERR_SHAPE, "n=%lld must be a non-negative multiple of 128", (long long)n);
  if (!x || !codes || !scale || !workspace) return fail(MOE_ERR_NULL, "x, codes, scale, workspace are required");
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(workspace, 16) || !aligned(scale, 4) ||
      !aligned(static_scale, 4))
    return fail(MOE_ERR_ALIGN, "x, codes and workspace must be 16-byte aligned");
  if (workspace_bytes < MOE_QUANT_WORKSPACE_BYTES)
    return fail(MOE_ERR_WORKSPACE, "workspace of %d bytes needed", MOE_QUANT_WORKSPACE_BYTES);
  if (n == 0) return ok();
  char* ws = (char*)workspace;
  int err = moe::launch_quant_x(x, x_dtype, (size_t)n, static_scale, (float*)ws, codes, scale,
                                (uint32_t*)(ws + moe::kMaxPartials * sizeof(float)),
                                (hipStream_t)stream);
  return hip_status(err, "quantisation launch");
}

}  // extern "C"
