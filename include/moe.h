/*
 * moe.h -- C ABI of the MI355X (gfx950) fused Mixture-of-Experts layer.
 *
 * Pages cited (titles as published):
 *   [post]    "Amazon SageMaker AI 上的 Mixture-of-Experts 内核工程优化"
 *             (English text of the AWS Machine Learning Blog post).
 *   [digest]  "AWS公布SageMaker AI上MoE融合内核的三项优化，H200吞吐提升最高 10%".
 *   [faq]     uniquestudio AI-news digest of the same post.
 *
 * The layer is one batched device operation made of three calls, issued in
 * this order on one stream: moe_route_topk -> moe_align_permute ->
 * moe_fused_forward ([post], introduction: routing, shuffling and the expert
 * networks merged into one batched op instead of a per-expert loop).
 *
 * Naming follows the expert GEMM statement A[M,K] x B[K,N] -> C[M,N] of
 * [post], "Swap-AB for WGMMA utilization": M = token rows (T), K = hidden
 * features (H), N = per-expert intermediate size (I; the gate/up projection
 * emits 2N).  Weights are passed already transposed, B^T[N,K] with K
 * contiguous ([faq], "背景与事实", the B^T[N,K] x A^T[K,M] form):
 *   w13 [E][2N][K]  rows [0,N) gate, rows [N,2N) up;   w2 [E][K][N].
 *
 * Conventions shared by every call:
 *   - Pointers named as device buffers are device pointers (hipMalloc or
 *     torch CUDA tensors), row-major and densely packed; activations,
 *     weights, outputs and workspaces 16-byte aligned, index, weight-of-
 *     routing and scale buffers 4-byte aligned (MOE_ERR_ALIGN otherwise).  The
 *     caller allocates and owns every buffer, including the workspace; the
 *     library keeps no pointer after returning and never allocates, frees,
 *     synchronises or reads device memory from the host.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).  All
 *     work is enqueued on it asynchronously; the calls can be captured into a
 *     HIP graph.  The token count M is only ever a kernel argument: no call
 *     compiles, allocates or waits for a new M (the lesson of [post], "Triton
 *     JIT recompilation elimination").
 *   - Every argument is validated on the host before anything is launched; a
 *     non-zero status means nothing was enqueued.  MOE_ERR_HIP means a launch
 *     was rejected by the runtime.  Faults inside kernels surface at the
 *     caller's next synchronisation.  moe_last_error() describes the last
 *     failure of the calling thread.
 *   - M == 0 is valid: after the size checks the call returns MOE_OK and
 *     enqueues nothing (buffers may then be NULL), except where documented.
 *   - Calls are reentrant and keep no state between calls (the one-time
 *     set-up of a kernel's LDS limit per device is thread-safe); concurrent
 *     calls must not share output or workspace buffers.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  MOE_ERR_DTYPE = 3,       /* an unknown dtype code */
  MOE_ERR_ALIGN = 4,       /* a pointer is not aligned as required */
  MOE_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  MOE_ERR_UNSUPPORTED = 6, /* valid values the library does not handle */
  MOE_ERR_HIP = 7          /* the HIP runtime rejected a launch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Problem description for moe_workspace_size / moe_fused_forward.
 *   M        token rows T, >= 0.
 *   K        hidden size H, multiple of 128, <= 65536.
 *   N        expert intermediate size I, multiple of 128, <= 65536.
 *   E        experts, 1..1024.
 *   topk     experts per token, 1..min(E, 64).
 *   block_m  segment padding used by moe_align_permute: 16, 32, 64, 128, 256.
 *   a_dtype  activations x: MOE_F32 or MOE_BF16; or, with E4M3 weights,
 *            MOE_FP8_E4M3: codes made beforehand (moe_quantize_act), their
 *            scale s_x in a1_scale (required), so that the quantisation can
 *            run beside the routing.
 *   w_dtype  weights: MOE_F32, MOE_BF16 (computed on bf16 MFMA, fp32
 *            accumulate; f32 values are rounded to bf16 on load) or
 *            MOE_FP8_E4M3 (OCP E4M3FN codes with one fp32 scale per expert
 *            and matrix; activations are then quantised to E4M3 per tensor,
 *            [post], "Backend routing for FP8 tensor quantization").
 *   out_dtype  MOE_F32 or MOE_BF16. */
typedef struct {
  int32_t M, K, N, E, topk, block_m;
  int32_t a_dtype, w_dtype, out_dtype;
} moe_problem;

/* Human-readable name of a status code (static string). */
const char* moe_status_string(int32_t status);

/* Description of the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

/* Upper bound of the padded pair list: P + min(E, P) * (block_m - 1) with
 * P = M * topk.  Returns -1 for invalid arguments.  Host only. */
int64_t moe_align_capacity(int32_t M, int32_t topk, int32_t E, int32_t block_m);

/* Bytes of device workspace that moe_align_permute and moe_fused_forward
 * need for problem *p (one buffer serves both calls; its contents need no
 * initialisation and are not preserved between calls).  Host only. */
moe_status moe_workspace_size(const moe_problem* p, size_t* bytes);

/* After moe_fused_forward with E4M3 weights has run, the workspace holds the
 * two per-tensor activation scales it applied, s_x then s_h, as fp32 at this
 * byte offset (until the workspace is next used).  Read-only for callers; a
 * diagnostic, not an input. */
#define MOE_WORKSPACE_SCALES_OFFSET 4096

/*
 * Top-k routing ([post], introduction, "token routing"; k experts per token,
 * uniquestudio digest, "背景与事实").  For every token row t:
 *   ids[t, 0:k]  the k expert ids with the largest logits, in descending
 *                logit order; equal logits go to the lower expert id
 *                (-0.0 and +0.0 are equal).  Selection compares the raw fp32
 *                logits, so ids are exact.
 *   w[t, j]      softmax probability of ids[t,j] in fp32; with
 *                renormalize != 0 divided by the sum over the k selected.
 * logits     device f32 [M, E]; finite values (NaN/Inf give unspecified ids).
 * topk_ids   device int32 [M, topk]  (written).
 * topk_weights device f32 [M, topk]  (written).
 * Limits: 1 <= E <= 1024, 1 <= topk <= min(E, 64), M >= 0.
 */
moe_status moe_route_topk(const float* logits, int32_t M, int32_t E,
                          int32_t topk, int32_t renormalize, int32_t* topk_ids,
                          float* topk_weights, void* stream);

/*
 * Per-expert token bucketing ([post], "Backend routing for FP8 tensor
 * quantization": small, fragmented token groups mapped onto the active
 * experts' weights).  Stable counting sort of the P = M*topk flat pair
 * indices f = t*topk + j by expert id:
 *   expert_offsets [E+1]  exclusive prefix sum of the padded counts
 *                         q_e = ceil(c_e / block_m) * block_m (0 if c_e = 0).
 *   sorted_pair_ids [cap] expert e's pairs at [offsets[e], offsets[e]+c_e)
 *                         in ascending f, then the sentinel P up to
 *                         offsets[e+1].  Entries at or past *num_padded are
 *                         unspecified.  cap = moe_align_capacity(...).
 *   block_expert_ids [cap / block_m]  expert of each block_m-row block
 *                         (defined for blocks below *num_padded / block_m).
 *   pair_pos [P]          position of pair f in sorted_pair_ids; -1 for a
 *                         pair whose id lies outside [0, E) (such pairs are
 *                         dropped from every segment).
 *   num_padded [1]        sum of q_e.
 * All outputs are device int32 buffers; topk_ids is device int32 [M, topk].
 * workspace: device, >= moe_workspace_size() bytes for a problem with these
 * M, topk, E, block_m (it may be NULL when M*topk <= 1024).  The result is
 * identical on every run.  M == 0 still writes expert_offsets (all 0) and
 * num_padded (0).
 */
moe_status moe_align_permute(const int32_t* topk_ids, int32_t M, int32_t topk,
                             int32_t E, int32_t block_m,
                             int32_t* sorted_pair_ids,
                             int32_t* block_expert_ids,
                             int32_t* expert_offsets, int32_t* pair_pos,
                             int32_t* num_padded, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * moe_route_topk followed by moe_align_permute, with the same arguments and
 * results as the two calls (bit for bit).  When M <= 8 and M*topk <= 1024
 * both run in one workgroup of one launch (one token row per wave), the ids
 * staying on chip between them; this is the small-decode case, where the
 * fixed cost of a launch is a visible part of the layer's time.  Larger
 * batches take the two-call path.
 */
moe_status moe_route_align(const float* logits, int32_t M, int32_t E, int32_t topk,
                           int32_t renormalize, int32_t block_m, int32_t* topk_ids,
                           float* topk_weights, int32_t* sorted_pair_ids,
                           int32_t* block_expert_ids, int32_t* expert_offsets,
                           int32_t* pair_pos, int32_t* num_padded, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Token routing from the hidden states: a linear router projection followed
 * by the routing of moe_route_topk ([post], introduction, "token routing";
 * the pages give no router formula, and this call reads it as a linear
 * router with one weight row per expert):
 *   logits[t, e] = sum_k x[t, k] * w_router[e, k]   (fp32 accumulation of
 *                  bf16 products; f32 inputs are rounded to bf16 first)
 * then ids and weights exactly as moe_route_topk computes them from these
 * fp32 logits.  Selection follows the fp32 logits, so where two logits lie
 * within the projection's rounding of each other the ids may differ from an
 * exact-arithmetic router.  The projection is split over K across the chip;
 * the slices are added in a fixed order, so the result is identical on
 * every run.
 * x          device [M, K] row-major, x_dtype MOE_BF16 or MOE_F32.
 * w_router   device [E, K] row-major (the router weight transposed, like
 *            w13 and w2: the hidden dimension contiguous), w_dtype == x_dtype.
 * logits     device f32 [M, E] (written) or NULL.
 * topk_ids, topk_weights: as moe_route_topk (written).
 * workspace  device, >= moe_route_project_workspace_size() bytes, 16-byte
 *            aligned (partial sums; no initialisation, not preserved).
 * Limits: K a multiple of 128 in [128, 65536]; E, topk, M as moe_route_topk.
 * x and w_router 16-byte aligned, the outputs 4-byte aligned.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE (a type other than
 * bf16 or f32), MOE_ERR_UNSUPPORTED (x_dtype != w_dtype), MOE_ERR_ALIGN,
 * MOE_ERR_WORKSPACE, MOE_ERR_HIP; nothing is enqueued on an error.  M == 0
 * is a no-op.
 */
moe_status moe_route_project_topk(const void* x, int32_t x_dtype, const void* w_router,
                                  int32_t w_dtype, int32_t M, int32_t K, int32_t E,
                                  int32_t topk, int32_t renormalize, float* logits,
                                  int32_t* topk_ids, float* topk_weights, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Bytes of workspace moe_route_project_topk needs for M tokens, hidden size
 * K and E experts (at most M * E * K / 32 bytes).  Host only. */
moe_status moe_route_project_workspace_size(int32_t M, int32_t K, int32_t E, size_t* bytes);

/*
 * Expert computation and weighted combine.  For each real pair (t, j) with
 * e = expert of the pair:
 *   g = x_t . w13[e, 0:N]^T,  u = x_t . w13[e, N:2N]^T,  h = SiLU(g) * u,
 *   y = h . w2[e]^T,          out[t] = sum_j topk_weights[t, j] * y
 * with SiLU(z) = z / (1 + exp(-z)), fp32 accumulation, h held in bf16
 * (bf16/f32 weights) or fp32 (E4M3 weights), the routing weight applied in
 * the fp32 epilogue of the down projection, and one bf16/f32 rounding of out.
 *
 * FP8 (w_dtype == MOE_FP8_E4M3), per-tensor scaling ([post], "Backend routing
 * for FP8 tensor quantization"; E4M3 named in "Amazon SageMaker AI 上的 MoE
 * 内核工程优化实践", "Triton 后端路由"):
 *   s_x = a1_scale ? *a1_scale : fl32(amax|x| / 448)  (1 if amax == 0),
 *   x codes = E4M3(fl32(x / s_x)), round to nearest even, saturating;
 *   GEMM1 output scaled by s_x * w13_scale[e];
 *   s_h = a2_scale ? *a2_scale : fl32(amax|h| / 448) over all real pairs,
 *   h codes = E4M3(fl32(h / s_h)), the correctly rounded fp32 quotient;
 *   GEMM2 output scaled by s_h * w2_scale[e].
 *
 * a      device [M, K] of a_dtype.       w13  device [E, 2N, K] of w_dtype.
 * w2     device [E, K, N] of w_dtype.    out  device [M, K] of out_dtype
 *        (must not alias any input).
 * w13_scale, w2_scale  device f32 [E]; required for E4M3 weights, else NULL.
 * a1_scale, a2_scale   device f32 [1] static scales or NULL (dynamic); only
 *        read for E4M3 weights.  With E4M3 activations a1_scale is required
 *        and is their scale s_x (the x quantisation is then skipped).
 * topk_weights         device f32 [M, topk] from moe_route_topk.
 * sorted_pair_ids, block_expert_ids, expert_offsets, pair_pos, num_padded
 *        device int32, from moe_align_permute with the same M, topk, E and
 *        p->block_m.
 * workspace            device, >= moe_workspace_size(p) bytes.
 */
moe_status moe_fused_forward(
    const moe_problem* p, const void* a, const void* w13, const void* w2,
    const float* w13_scale, const float* w2_scale, const float* a1_scale,
    const float* a2_scale, const float* topk_weights,
    const int32_t* sorted_pair_ids, const int32_t* block_expert_ids,
    const int32_t* expert_offsets, const int32_t* pair_pos,
    const int32_t* num_padded, void* out, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * FP8 activation quantisation on its own (the step moe_fused_forward runs
 * first for E4M3 weights; exposed so that callers can pre-quantise and tests
 * can check the codes bit for bit).  Per-tensor scaling as in [post],
 * "Backend routing for FP8 tensor quantization":
 *   *scale = static_scale ? *static_scale : fl32(amax|x| / 448) (1 if 0);
 *   codes[i] = E4M3(fl32(x[i] / *scale)) (the correctly rounded fp32 quotient), round to
 *   nearest even, saturating at +-448 (OCP E4M3FN).
 * x          device [n] of x_dtype (MOE_F32 or MOE_BF16), 16-byte aligned.
 * n          element count, a multiple of 128, >= 0.
 * codes      device uint8 [n] (written), 16-byte aligned.
 * scale      device f32 [1] (written).
 * workspace  device, >= MOE_QUANT_WORKSPACE_BYTES bytes, 16-byte aligned.
 */
#define MOE_QUANT_WORKSPACE_BYTES 8192
moe_status moe_quantize_act(const void* x, int32_t x_dtype, int64_t n,
                            const float* static_scale, uint8_t* codes,
                            float* scale, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * moe_fused_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and errors, without the
 * workspace arguments.  The workspace is a device array inside the library,
 * MOE_NOALLOC_SCRATCH_BYTES per device, held from the first call on a device
 * until the process ends; the call itself allocates nothing.  Problems whose
 * moe_workspace_size exceeds it are rejected with MOE_ERR_WORKSPACE (the
 * decode shapes of H = 4096, I = 1024, E = 64, top-8 up to M = 64, bf16 or
 * E4M3 weights, need about 20 MiB).  Every call on a device uses that
 * device's one array: calls that overlap in time on one device (several
 * streams or threads) race and must be serialised by the caller.  The array
 * needs no initialisation; after an E4M3 call it holds s_x and s_h at
 * MOE_WORKSPACE_SCALES_OFFSET like a caller workspace.  The device is the
 * current one; `stream` must belong to it.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_fused_forward_noalloc(
    const moe_problem* p, const void* a, const void* w13, const void* w2,
    const float* w13_scale, const float* w2_scale, const float* a1_scale,
    const float* a2_scale, const float* topk_weights,
    const int32_t* sorted_pair_ids, const int32_t* block_expert_ids,
    const int32_t* expert_offsets, const int32_t* pair_pos,
    const int32_t* num_padded, void* out, void* stream);

/*
 * moe_fused_forward for E4M3 decode batches in one kernel launch: the
 * pages' single hardware pass of the FP8 path, in which scaling, the expert
 * GEMMs and the aggregation run as one fused step instead of discrete
 * kernels with HBM round trips in between ([post], "Backend routing for FP8
 * tensor quantization"; "Amazon SageMaker AI 上的 MoE 内核工程优化实践",
 * "Triton 后端路由").  The same computation as moe_fused_forward, with its
 * arguments and errors, and the same result bit for bit (every step is done
 * in the same arithmetic).  One persistent grid of two workgroups per CU runs
 * the steps as phases separated by grid-wide barriers: the activation scale
 * and codes, gate/up with SiLU * up, the scale and codes of h, the down
 * projection, and the weighted combine, which the workgroup finishing the
 * last expert block of each 32-row output block performs.  After the
 * workspace arguments:
 * sync       device, >= MOE_FUSED_SYNC_BYTES bytes, 128-byte aligned: the
 *            barrier words.  Zero it once before the first call (every call
 *            leaves it in a state the next call starts from); keep one per
 *            stream: calls that overlap in time on one sync buffer race.
 *            After a call, the 32-bit word at byte offset
 *            MOE_FUSED_SYNC_ERROR_OFFSET is nonzero if a grid-wide wait gave
 *            up (after about a second: the grid's workgroups could not all
 *            be resident at once, e.g. when another kernel held the CUs);
 *            that call's output is then undefined and the buffer must be
 *            zeroed again.
 * Limits beyond moe_fused_forward's: w_dtype MOE_FP8_E4M3, a_dtype bf16 or
 * f32, 1 <= M <= 64 (M == 0 is a no-op), p->block_m == 16, and byte
 * offsets of the per-pair buffers below 4 GiB; otherwise
 * MOE_ERR_UNSUPPORTED.  MOE_ERR_HIP also when the device cannot hold two
 * workgroups per CU of this kernel.
 */
#define MOE_FUSED_SYNC_BYTES 32768
#define MOE_FUSED_SYNC_ERROR_OFFSET 128
moe_status moe_fused_forward_persistent(
    const moe_problem* p, const void* a, const void* w13, const void* w2,
    const float* w13_scale, const float* w2_scale, const float* a1_scale,
    const float* a2_scale, const float* topk_weights,
    const int32_t* sorted_pair_ids, const int32_t* block_expert_ids,
    const int32_t* expert_offsets, const int32_t* pair_pos,
    const int32_t* num_padded, void* out, void* workspace,
    size_t workspace_bytes, void* sync, size_t sync_bytes, void* stream);

/*
 * moe_fused_forward with timing events: the same computation, arguments and
 * errors, and in addition hipEventRecord of events[0] / events[1] (hipEvent_t
 * passed as void*) on `stream` right before and after the gate/up GEMM
 * launch, and of events[2] / events[3] around the down GEMM launch (for
 * M <= 64 with f32 weights that launch also does the combine; otherwise the
 * combine kernel runs after events[3]).  NULL entries, or events == NULL,
 * are skipped.  Under stream capture each record is added to the graph as
 * an event-record node, so every replay re-records the event at that point.
 * A failed record returns MOE_ERR_HIP.  For measuring kernel durations; no
 * state is kept.
 */
moe_status moe_fused_forward_profiled(
    const moe_problem* p, const void* a, const void* w13, const void* w2,
    const float* w13_scale, const float* w2_scale, const float* a1_scale,
    const float* a2_scale, const float* topk_weights,
    const int32_t* sorted_pair_ids, const int32_t* block_expert_ids,
    const int32_t* expert_offsets, const int32_t* pair_pos,
    const int32_t* num_padded, void* out, void* workspace,
    size_t workspace_bytes, void* stream, void* const events[4]);

/*
 * Rotary position embedding fused with per-head FP8 quantisation: the kernel
 * that the AWS post names in "Triton JIT recompilation elimination" (rotary
 * position embedding and FP8 quantisation fused, per head), whose token count
 * must never trigger a recompile.  The pages give no formula; this call reads
 * it as follows, for x [T, n_heads, head_dim] (D = head_dim):
 *   angle a(t, i) = fl32(positions[t] * inv_freq[i]), i < D/2, negated when
 *     `inverse` (the rotation back);
 *   pairs (x[t,h,i], x[t,h,i+D/2]) (interleaved == 0) or
 *     (x[t,h,2i], x[t,h,2i+1]) (interleaved != 0); (u, v) becomes
 *     (u cos a - v sin a, v cos a + u sin a), computed in fp32;
 *   one scale per head over the call's T tokens:
 *     scales[h] = static_scales ? static_scales[h]
 *                               : fl32(amax over t, d of |y[t,h,d]| / 448)
 *     (1 when that amax is 0);
 *   codes[t,h,d] = E4M3(fl32(y[t,h,d] / scales[h])), round to nearest even,
 *     saturating at +-448 (OCP E4M3FN).
 * x          device [T, n_heads, head_dim] of x_dtype (MOE_BF16 or MOE_F32),
 *            16-byte aligned.
 * positions  device int32 [T], |positions[t]| < 2^24.
 * inv_freq   device f32 [head_dim / 2] (e.g. base^(-2i/D)).
 * static_scales  device f32 [n_heads] or NULL (dynamic); normal positive values.
 * codes      device uint8 [T, n_heads, head_dim] (written), 16-byte aligned.
 * scales     device f32 [n_heads] (written: the scales used).
 * workspace  device, >= moe_rope_workspace_size() bytes, 16-byte aligned (no
 *            initialisation, not preserved).
 * Limits: 1 <= n_heads <= 256; head_dim a multiple of 16 in [16, 512].
 * T == 0 is a no-op.  Errors: MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_NULL,
 * MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_HIP; nothing is enqueued on an
 * error.  T is only ever a kernel argument.
 */
moe_status moe_rope_quantize_per_head(const void* x, int32_t x_dtype, const int32_t* positions,
                                      const float* inv_freq, int32_t T, int32_t n_heads,
                                      int32_t head_dim, int32_t interleaved, int32_t inverse,
                                      const float* static_scales, uint8_t* codes, float* scales,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace moe_rope_quantize_per_head needs.  Host only. */
moe_status moe_rope_workspace_size(int32_t T, int32_t n_heads, int32_t head_dim, size_t* bytes);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
