/*
 * moe_oracle.c -- plain, slow, fp64 CPU oracle for the fused MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no source, header,
 * table or helper with the GPU library; it reads the same input bytes.
 *
 * Pages cited (titles as published):
 *   [post]    "Amazon SageMaker AI 上的 Mixture-of-Experts 内核工程优化"
 *             (English text of the AWS Machine Learning Blog post).
 *   [digest]  "AWS公布SageMaker AI上MoE融合内核的三项优化，H200吞吐提升最高 10%".
 *   [comment] "Amazon SageMaker AI 上的 MoE 内核工程优化实践".
 *   [faq]     uniquestudio AI-news digest of the same post ("背景与事实").
 *
 * What the pages fix: a fused MoE op routes tokens, shuffles them per expert,
 * runs the expert networks and aggregates, as one batched op ([post],
 * introduction; [digest], summary).  Routing is dynamic with k experts per
 * token, topk=8 in the example ([comment], "为什么 MoE 推理…"; [faq], "背景与
 * 事实").  The expert product is A[M,K] x B[K,N] with M token rows, K hidden
 * features and N the expert output dimension ([post], "Swap-AB for WGMMA
 * utilization").  FP8 per-tensor scaling is applied around the expert GEMMs
 * and the expert aggregation ([post], "Backend routing for FP8 tensor
 * quantization").  FP8 E4M3 has 4 exponent and 3 mantissa bits ([comment],
 * "Triton 后端路由").
 *
 * What the pages leave open, and the reading taken here (each one is also
 * listed in the design notes):
 *   - the linear router of oracle_route_project: logits = x . W_r^T with
 *     W_r [E, K] (hidden dimension contiguous), selection on the fp64 logits;
 *   - logits are an input; selection is on the raw fp32 logits, descending,
 *     ties to the lower expert id; weights are the softmax of the logits
 *     (fp64), renormalised over the k selected when asked;
 *   - rows [0,I) of w13[e] are the gate (SiLU side), rows [I,2I) the up side;
 *     SiLU(z) = z / (1 + exp(-z));
 *   - the routing weight multiplies the down-projection output;
 *   - per-expert alignment pads each expert segment to a multiple of block_m,
 *     lists its pair indices f = t*k + j ascending, fills with sentinel P;
 *   - E4M3 is the OCP E4M3FN format (max 448, codes 0x7F/0xFF are NaN);
 *     encoding rounds to nearest, ties to even, saturating at +-448;
 *   - activation scale s = fl32(amax / 448) (1 when amax = 0); the code of x
 *     is E4M3(fl32(x / s)) with an IEEE fp32 division;
 *   - rotary position embedding with per-head E4M3 quantisation
 *     (oracle_rope_quant_per_head): the inverse-frequency table is an input,
 *     the angle of pair i of token t is fl32(pos[t] * inv_freq[i]), the pair
 *     is rotated by that angle (by its negative when `inverse`), pairs are
 *     (i, i + D/2) or (2i, 2i + 1); one scale per head over the call's tokens;
 *   - the intermediate h is quantised with one dynamic scale over all real
 *     pairs, the same per-tensor rule as x: s_h = fl32(amax|h| / 448) with
 *     amax taken over the fp64 values; its code is E4M3(fl32(h / s_h)), the
 *     quotient formed in fp64 and rounded once to binary32 (the precision in
 *     which the encoding decision is taken).
 *
 * Parity unpinned: the element-level codes of the FP8 intermediate h.  The GPU
 * holds h in fp32 after its own summation order, so an element close to a
 * rounding boundary may land one E4M3 step away; only the end-to-end error
 * bound covers it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_E4M3 2

/* ---------------------------------------------------------------- codecs */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
double oracle_bf16_to_f64(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinity,
 * S.1111.111 is NaN.  Normal: (1 + m/8) * 2^(e-7); subnormal: (m/8) * 2^-6.
 * The format is named in [comment], "Triton 后端路由". */
double oracle_e4m3_to_f64(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest E4M3FN code to a binary32 value: search every finite magnitude
 * code, keep the closest; on an exact tie keep the even code (round half to
 * even).  Magnitudes at or beyond 448 saturate to 448.  NaN maps to 0x7F. */
static double g_e4m3_mag[0x7F];
static int g_e4m3_ready = 0;

uint8_t oracle_e4m3_from_f32(float f) {
  if (!g_e4m3_ready) { /* magnitudes of codes 0x00..0x7E (idempotent fill) */
    for (int c = 0; c < 0x7F; ++c) g_e4m3_mag[c] = oracle_e4m3_to_f64((uint8_t)c);
    g_e4m3_ready = 1;
  }
  if (isnan(f)) return 0x7F;
  uint8_t sign = signbit(f) ? 0x80 : 0x00;
  double a = fabs((double)f);
  if (a >= 448.0) return sign | 0x7E;
  int best = 0;
  double best_d = a; /* distance to code 0 */
  for (int c = 1; c <= 0x7E; ++c) {
    double d = fabs(a - g_e4m3_mag[c]);
    if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_d = d;
    }
  }
  return sign | (uint8_t)best;
}

/* Values of all 256 E4M3 codes, filled once from oracle_e4m3_to_f64 (a
 * lookup of the same numbers, so that the expert loops need not re-derive
 * each weight's value). */
static double g_e4m3_val[256];
static int g_e4m3_val_ready = 0;

static void fill_tables(void) {
  if (!g_e4m3_val_ready) {
    for (int c = 0; c < 256; ++c) g_e4m3_val[c] = oracle_e4m3_to_f64((uint8_t)c);
    g_e4m3_val_ready = 1;
  }
  (void)oracle_e4m3_from_f32(0.0f); /* the encoder's table */
}

static double load_elem(int dtype, const void* p, int64_t i) {
  switch (dtype) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_BF16: return oracle_bf16_to_f64(((const uint16_t*)p)[i]);
    default: return g_e4m3_val[((const uint8_t*)p)[i]];
  }
}

/* ---------------------------------------------------------------- routing */

typedef struct {
  float v;
  int id;
} orc_cand;

/* Order: larger logit first; equal logits (including -0 vs +0) by lower id. */
static int cand_cmp(const void* pa, const void* pb) {
  const orc_cand* a = (const orc_cand*)pa;
  const orc_cand* b = (const orc_cand*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

/* Top-k routing of one batch of logits [T,E] (row-major).  Dynamic routing of
 * each token to k experts: [comment], "为什么 MoE 推理对内核工程如此敏感";
 * topk=8 example: [faq], "背景与事实".  Weights in fp64. */
int oracle_route_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                      int32_t renormalize, int32_t* ids, double* w) {
  if (T < 0 || E < 1 || k < 1 || k > E) return 1;
  orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)E);
  if (!c) return 2;
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    for (int e = 0; e < E; ++e) {
      c[e].v = l[e];
      c[e].id = e;
    }
    qsort(c, (size_t)E, sizeof(orc_cand), cand_cmp);
    double m = (double)c[0].v;
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += exp((double)l[e] - m);
    double zs = 0.0;
    for (int j = 0; j < k; ++j) zs += exp((double)c[j].v - m);
    for (int j = 0; j < k; ++j) {
      double p = exp((double)c[j].v - m);
      ids[t * k + j] = c[j].id;
      w[t * k + j] = renormalize ? p / zs : p / z;
    }
  }
  free(c);
  return 0;
}

/* ------------------------------------------------------ router projection */

typedef struct {
  double v;
  int id;
} orc_cand64;

static int cand64_cmp(const void* pa, const void* pb) {
  const orc_cand64* a = (const orc_cand64*)pa;
  const orc_cand64* b = (const orc_cand64*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

/* Token routing from the hidden states themselves.  The pages name token
 * routing as the first stage the fused op takes over ([post], introduction;
 * [digest], summary) but give no router formula.  Reading taken here: a
 * linear router with one weight row per expert, stored like the expert
 * weights with the hidden dimension contiguous (W_r [E, K]):
 *   logits[t, e] = sum_k x[t, k] * W_r[e, k]      (fp64 over the stored values)
 * then the selection and weights of oracle_route_topk on these fp64 logits
 * (descending, ties to the lower id; softmax, renormalised over the k when
 * asked).  x and W_r are f32 or bf16 (dtype codes). */
int oracle_route_project(int x_dtype, const void* x, int w_dtype, const void* wr, int64_t T,
                         int32_t K, int32_t E, int32_t k, int32_t renormalize, double* logits,
                         int32_t* ids, double* w) {
  fill_tables();
  if (T < 0 || K < 1 || E < 1 || k < 1 || k > E) return 1;
  if ((x_dtype != ORC_F32 && x_dtype != ORC_BF16) || (w_dtype != ORC_F32 && w_dtype != ORC_BF16))
    return 3;
  orc_cand64* c = (orc_cand64*)malloc(sizeof(orc_cand64) * (size_t)E);
  if (!c) return 2;
  for (int64_t t = 0; t < T; ++t) {
    double* l = logits + t * E;
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int32_t kk = 0; kk < K; ++kk)
        acc += load_elem(x_dtype, x, t * K + kk) * load_elem(w_dtype, wr, (int64_t)e * K + kk);
      l[e] = acc;
      c[e].v = acc;
      c[e].id = e;
    }
    qsort(c, (size_t)E, sizeof(orc_cand64), cand64_cmp);
    double m = c[0].v;
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += exp(l[e] - m);
    double zs = 0.0;
    for (int j = 0; j < k; ++j) zs += exp(c[j].v - m);
    for (int j = 0; j < k; ++j) {
      double p = exp(c[j].v - m);
      ids[t * k + j] = c[j].id;
      w[t * k + j] = renormalize ? p / zs : p / z;
    }
  }
  free(c);
  return 0;
}

/* ---------------------------------------------------------------- align */

/* Counting sort of the P = T*k flat pair indices by expert, each expert's
 * segment padded to a multiple of block_m with the sentinel P.  This is the
 * per-expert token bucketing of [post], "Backend routing for FP8 tensor
 * quantization" (small, fragmented token groups mapped onto the active
 * experts' weights).  Out-of-range ids are not placed and get pair_pos -1. */
int oracle_align(const int32_t* ids, int64_t T, int32_t k, int32_t E,
                 int32_t block_m, int32_t* sorted_pair_ids,
                 int32_t* block_expert_ids, int32_t* expert_offsets,
                 int32_t* pair_pos, int32_t* num_padded) {
  if (T < 0 || k < 1 || E < 1 || block_m < 1) return 1;
  int64_t P = T * (int64_t)k;
  int64_t* cnt = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* fill = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  if (!cnt || !fill) return 2;
  for (int64_t f = 0; f < P; ++f)
    if (ids[f] >= 0 && ids[f] < E) cnt[ids[f]]++;
  int64_t off = 0;
  for (int e = 0; e < E; ++e) {
    expert_offsets[e] = (int32_t)off;
    int64_t q = (cnt[e] + block_m - 1) / block_m * block_m;
    for (int64_t s = off; s < off + q; ++s) sorted_pair_ids[s] = (int32_t)P;
    for (int64_t b = off / block_m; b < (off + q) / block_m; ++b)
      block_expert_ids[b] = e;
    off += q;
  }
  expert_offsets[E] = (int32_t)off;
  *num_padded = (int32_t)off;
  for (int64_t f = 0; f < P; ++f) {
    int e = ids[f];
    if (e < 0 || e >= E) {
      pair_pos[f] = -1;
      continue;
    }
    int64_t pos = expert_offsets[e] + fill[e]++;
    sorted_pair_ids[pos] = (int32_t)f;
    pair_pos[f] = (int32_t)pos;
  }
  free(cnt);
  free(fill);
  return 0;
}

/* ------------------------------------------------- FP8 per-tensor scaling */

/* Dynamic per-tensor scale: fl32(amax / 448), 1 when amax == 0.  The
 * per-tensor FP8 scaling is the scheme of [post], "Backend routing for FP8
 * tensor quantization"; 448 is the largest finite E4M3FN magnitude. */
float oracle_act_scale(int dtype, const void* x, int64_t n) {
  fill_tables();
  double amax = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double v = fabs(load_elem(dtype, x, i));
    if (v > amax) amax = v;
  }
  if (amax == 0.0) return 1.0f;
  return (float)amax / 448.0f;
}

/* code = E4M3(fl32(x / s)), the division done in IEEE binary32. */
void oracle_quantize_e4m3(int dtype, const void* x, int64_t n, float s,
                          uint8_t* q) {
  fill_tables();
  for (int64_t i = 0; i < n; ++i) {
    float v = (float)load_elem(dtype, x, i);
    q[i] = oracle_e4m3_from_f32(v / s);
  }
}

/* --------------------------------------------------------------- forward */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert's gate/up projection and gating for one token row:
 * a_i = SiLU(sum_h W13[e,i,h] x_h) * (sum_h W13[e,I+i,h] x_h). */
static void expert_gate_up(int w_dtype, const void* w13, double w13s, int64_t e,
                           int32_t H, int32_t I, const double* x, double* a) {
  for (int32_t i = 0; i < I; ++i) {
    int64_t rg = (e * 2 * (int64_t)I + i) * H;
    int64_t ru = (e * 2 * (int64_t)I + I + i) * H;
    double g = 0.0, u = 0.0;
    for (int32_t h = 0; h < H; ++h) {
      g += load_elem(w_dtype, w13, rg + h) * w13s * x[h];
      u += load_elem(w_dtype, w13, ru + h) * w13s * x[h];
    }
    a[i] = silu(g) * u;
  }
}

/* One expert's down projection: y_n = sum_i W2[e,n,i] a_i. */
static void expert_down(int w_dtype, const void* w2, double w2s, int64_t e,
                        int32_t H, int32_t I, const double* a, double* y) {
  for (int32_t n = 0; n < H; ++n) {
    int64_t r = (e * (int64_t)H + n) * I;
    double acc = 0.0;
    for (int32_t i = 0; i < I; ++i)
      acc += load_elem(w_dtype, w2, r + i) * w2s * a[i];
    y[n] = acc;
  }
}

/*
 * Fused MoE forward, the layer the pages fuse into one batched op ([post],
 * introduction; expert aggregation and FP8 scaling: [post], "Backend routing
 * for FP8 tensor quantization").  For every requested token t and each of its
 * k routed experts e = ids[t,j], in fp64:
 *   g, u from w13[e]; a = SiLU(g) * u; y = W2[e] a; out[t] += w[t,j] * y.
 *
 * x: [T,H] (F32 or BF16).  w13: [E,2I,H]; w2: [E,H,I] (F32, BF16 or E4M3 with
 * per-expert scales w13_scale[E], w2_scale[E]).  fp8_act != 0 quantises x and
 * h per tensor (a1_scale / a2_scale override the dynamic scales when given).
 * ids/w: routing [T,k].  tokens: which rows to produce (NULL = all T, in
 * order); out: [n_tokens, H].  scales_out[0..1] receive the x and h scales
 * used (1 when not FP8).  Threads: OpenMP over (token, slot) pairs.
 */
int oracle_moe_forward(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k,
                       int32_t x_dtype, const void* x, int32_t w_dtype,
                       const void* w13, const void* w2, const float* w13_scale,
                       const float* w2_scale, int32_t fp8_act,
                       const float* a1_scale, const float* a2_scale,
                       const int32_t* ids, const double* w,
                       const int64_t* tokens, int64_t n_tokens, double* out,
                       float* scales_out) {
  fill_tables();
  if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1) return 1;
  if (w_dtype == ORC_E4M3 && (!w13_scale || !w2_scale)) return 1;
  int64_t P = T * (int64_t)k;
  if (!tokens) n_tokens = T;

  /* x as used by the expert GEMMs (dequantised when FP8). */
  double* xd = (double*)malloc(sizeof(double) * (size_t)(T * (int64_t)H + 1));
  if (!xd) return 2;
  float sx = 1.0f;
  if (fp8_act) {
    /* the scale spans all of x; rows are quantised where they are used */
    sx = a1_scale ? *a1_scale : oracle_act_scale(x_dtype, x, T * (int64_t)H);
    int need_all = !a2_scale || !tokens;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      int used = need_all;
      for (int64_t q = 0; !used && q < n_tokens; ++q) used = (tokens[q] == t);
      if (!used) continue;
      for (int32_t h = 0; h < H; ++h) {
        float v = (float)load_elem(x_dtype, x, t * H + h);
        xd[t * H + h] = (double)sx * oracle_e4m3_to_f64(oracle_e4m3_from_f32(v / sx));
      }
    }
  } else {
    for (int64_t i = 0; i < T * (int64_t)H; ++i)
      xd[i] = load_elem(x_dtype, x, i);
  }

  /* Pairs to evaluate: all pairs of the requested tokens. */
  int64_t np = n_tokens * k;
  double* a = (double*)malloc(sizeof(double) * (size_t)(np * I + 1));
  double* y = (double*)malloc(sizeof(double) * (size_t)(np * H + 1));
  if (!a || !y) return 2;

  float sh = 1.0f;
  if (fp8_act) {
    if (a2_scale) {
      sh = *a2_scale;
    } else {
      /* The h scale spans every real pair of the batch, not only the
       * requested tokens, so the gate/up pass runs over all T*k pairs. */
      double amax = 0.0;
#pragma omp parallel for schedule(dynamic, 1) reduction(max : amax)
      for (int64_t p = 0; p < P; ++p) {
        double* ta = (double*)malloc(sizeof(double) * (size_t)I);
        int64_t t = p / k;
        int e = ids[p];
        double s13 = (w_dtype == ORC_E4M3) ? (double)w13_scale[e] : 1.0;
        expert_gate_up(w_dtype, w13, s13, e, H, I, xd + t * H, ta);
        for (int32_t i = 0; i < I; ++i) {
          double v = fabs(ta[i]);
          if (v > amax) amax = v;
        }
        free(ta);
      }
      sh = (amax == 0.0) ? 1.0f : (float)(amax / 448.0);
    }
  }

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < np; ++p) {
    int64_t t = tokens ? tokens[p / k] : p / k;
    int j = (int)(p % k);
    int e = ids[t * k + j];
    double s13 = (w_dtype == ORC_E4M3) ? (double)w13_scale[e] : 1.0;
    double s2 = (w_dtype == ORC_E4M3) ? (double)w2_scale[e] : 1.0;
    double* pa = a + p * I;
    expert_gate_up(w_dtype, w13, s13, e, H, I, xd + t * H, pa);
    if (fp8_act) {
      for (int32_t i = 0; i < I; ++i) {
        float hv = (float)(pa[i] / (double)sh);
        pa[i] = (double)sh * oracle_e4m3_to_f64(oracle_e4m3_from_f32(hv));
      }
    }
    expert_down(w_dtype, w2, s2, e, H, I, pa, y + p * H);
  }

  /* Weighted top-k combine, slots in routing order. */
  for (int64_t q = 0; q < n_tokens; ++q) {
    int64_t t = tokens ? tokens[q] : q;
    for (int32_t n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += w[t * k + j] * y[(q * k + j) * H + n];
      out[q * H + n] = acc;
    }
  }
  if (scales_out) {
    scales_out[0] = sx;
    scales_out[1] = sh;
  }
  free(xd);
  free(a);
  free(y);
  return 0;
}

/* ------------------------------------------ rotary embedding + per-head FP8 */

/*
 * Rotary position embedding fused with per-head FP8 quantisation, the kernel
 * the AWS post names in "Triton JIT recompilation elimination" (rotary
 * position embedding and FP8 quantisation fused, per head).  The pages give no
 * formula; the reading taken here:
 *   x [T, nH, D] (f32 or bf16), D even; positions pos [T]; the inverse
 *   frequencies inv_freq [D/2] (fp32, an input: the "inv" table of RoPE,
 *   base^(-2i/D) in the usual construction).
 *   angle a(t, i) = fl32(pos[t] * inv_freq[i]), negated when `inverse`;
 *   each pair (u, v) of head h -- u = x[t,h,i], v = x[t,h,i + D/2] (halves),
 *   or u = x[t,h,2i], v = x[t,h,2i+1] (interleaved) -- becomes
 *     u' = u cos a - v sin a,   v' = v cos a + u sin a      (fp64);
 *   per head h: s_h = fl32(amax over t and d of |y[t,h,d]| / 448), 1 when the
 *   amax is 0, or static_scales[h] when given; codes E4M3(fl32(y / s_h)).
 * y_out (optional, fp64 [T, nH, D]) receives the rotated values.
 */
int oracle_rope_quant_per_head(int32_t x_dtype, const void* x, const int32_t* pos,
                               const float* inv_freq, int64_t T, int32_t nH, int32_t D,
                               int32_t interleaved, int32_t inverse, const float* static_scales,
                               uint8_t* codes, float* scales, double* y_out) {
  if (T < 0 || nH < 1 || D < 2 || D % 2) return 1;
  if (x_dtype != ORC_F32 && x_dtype != ORC_BF16) return 3;
  fill_tables();
  const int32_t half = D / 2;
  const int64_t n = T * (int64_t)nH * D;
  double* y = y_out ? y_out : (double*)malloc(sizeof(double) * (size_t)(n + 1));
  double* amax = (double*)calloc((size_t)nH, sizeof(double));
  if (!y || !amax) return 2;
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t i = 0; i < half; ++i) {
      float a32 = (float)((double)pos[t] * (double)inv_freq[i]);
      double a = inverse ? -(double)a32 : (double)a32;
      double c = cos(a), sn = sin(a);
      for (int32_t h = 0; h < nH; ++h) {
        int64_t base = (t * nH + h) * (int64_t)D;
        int64_t iu = base + (interleaved ? 2 * i : i);
        int64_t iv = base + (interleaved ? 2 * i + 1 : i + half);
        double u = load_elem(x_dtype, x, iu), v = load_elem(x_dtype, x, iv);
        y[iu] = u * c - v * sn;
        y[iv] = v * c + u * sn;
      }
    }
  }
  for (int64_t t = 0; t < T; ++t)
    for (int32_t h = 0; h < nH; ++h)
      for (int32_t d = 0; d < D; ++d) {
        double v = fabs(y[(t * nH + h) * (int64_t)D + d]);
        if (v > amax[h]) amax[h] = v;
      }
  for (int32_t h = 0; h < nH; ++h)
    scales[h] = static_scales ? static_scales[h]
                              : (amax[h] == 0.0 ? 1.0f : (float)(amax[h] / 448.0));
  for (int64_t t = 0; t < T; ++t)
    for (int32_t h = 0; h < nH; ++h)
      for (int32_t d = 0; d < D; ++d) {
        int64_t k = (t * nH + h) * (int64_t)D + d;
        codes[k] = oracle_e4m3_from_f32((float)(y[k] / (double)scales[h]));
      }
  if (!y_out) free(y);
  free(amax);
  return 0;
}
