"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI
binding, run the fp64 oracle on the same input bytes, compare."""
import numpy as np
import torch

import oracle
from mixture_experts_layer_13_amd import inputs, moe

BF16_TOL = 1e-2
FP8_TOL = 3e-2


def say(*a):
    print(*a, flush=True)


def row_rel_err(got, ref):
    """max over rows of max|g - r| / max|r| (rows with max|r| = 0 use abs)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if len(num) else 0.0


# Bound on |s_h(GPU) / s_h(oracle) - 1|.  The GPU forms each h element in
# fp32: E4M3 x E4M3 products are exact in fp32, and the fp32 accumulator
# takes one rounding per MFMA along K (K/64 = 64 at H = 4096, 112 at H =
# 7168), so the gate and up sums are each within about n * 2^-24 * sum|t| of
# the exact ones; at the element of largest |h| sum|t| / |sum t| is below
# about 10 for these inputs (x ~ N(0, 1), w ~ N(0, 0.02^2)), giving 112 *
# 2^-24 * 10 = 6.7e-5 per factor.  The dequant-scale product, SiLU and the
# division by 448 add a few ulps.  2^-12 covers both factors with margin.
SH_REL_TOL = 2.0 ** -12


def run_gpu(d, block_m=None, a1_scale=None, a2_scale=None, out_dtype=None, renormalize=True):
    """Whole layer on the GPU through the three ABI calls (block_m None: the
    layer's own default, as the benchmark runs it)."""
    x, logits, w13, w2 = d["x"], d["logits"], d["w13"], d["w2"]
    T, H, I, E, k = d["T"], d["H"], d["I"], d["E"], d["topk"]
    w = d["workload"]
    out_dtype = out_dtype or w.out_dtype
    bm = block_m
    dev = x.device
    a1 = None if a1_scale is None else torch.tensor([a1_scale], dtype=torch.float32, device=dev)
    a2 = None if a2_scale is None else torch.tensor([a2_scale], dtype=torch.float32, device=dev)
    layer = moe.FusedMoE(T, H, I, E, k, w13, w2, d["w13_scale"], d["w2_scale"], block_m=bm,
                         a_dtype=x.dtype, out_dtype=out_dtype, renormalize=renormalize,
                         a1_scale=a1, a2_scale=a2, device=dev)
    out = layer(x, logits)
    torch.cuda.synchronize()
    return layer, out


def oracle_forward(d, tokens=None, a1_scale=None, a2_scale=None, renormalize=True):
    """fp64 oracle on the same bytes; only the experts the oracle's own routing
    selects are copied to the host (ids remapped to the compact list)."""
    w = d["workload"]
    logits = d["logits"].cpu().numpy()
    ids, wts = oracle.route_topk(logits, d["topk"], renormalize)
    used = ids if tokens is None or (w.fp8_act and a2_scale is None) else ids[tokens]
    experts = np.unique(used)
    remap = np.full(d["E"], -1, np.int32)
    remap[experts] = np.arange(len(experts), dtype=np.int32)
    sel = torch.as_tensor(experts, device=d["w13"].device, dtype=torch.long)
    w13 = inputs.to_numpy_bits(d["w13"].index_select(0, sel))
    w2 = inputs.to_numpy_bits(d["w2"].index_select(0, sel))
    s13 = s2 = None
    if d["w13_scale"] is not None:
        s13 = d["w13_scale"].index_select(0, sel).cpu().numpy()
        s2 = d["w2_scale"].index_select(0, sel).cpu().numpy()
    ids_c = remap[ids]
    if (ids_c < 0).any() and tokens is not None:
        keep = np.zeros(len(ids), bool)
        keep[tokens] = True
        assert (ids_c[keep] >= 0).all()
        ids_c = np.where(ids_c < 0, 0, ids_c)
    out, scales = oracle.moe_forward(inputs.to_numpy_bits(d["x"]), w13, w2, ids_c, wts, s13, s2,
                                     fp8_act=w.fp8_act, a1_scale=a1_scale, a2_scale=a2_scale,
                                     tokens=tokens)
    return out, ids, wts, scales


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def sample_tokens(ids, n=256, seed=0):
    """Every token when T <= n; else the token of the last real pair of every
    expert segment (the largest flat index routed to each expert) plus a
    seeded random fill up to n, sorted."""
    T, k = ids.shape
    if T <= n:
        return np.arange(T)
    flat = ids.reshape(-1)
    uniq, first_rev = np.unique(flat[::-1], return_index=True)
    last_pairs = flat.size - 1 - first_rev
    toks = set((last_pairs // k).tolist())
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(T), np.fromiter(toks, np.int64))
    toks.update(rng.choice(rest, size=max(0, n - len(toks)), replace=False).tolist())
    return np.array(sorted(toks), np.int64)


def oracle_h_scale(d, ids):
    """(s_x, s_h) of the oracle over every real pair of the batch (all-pairs
    gate/up as fp64 library matmuls)."""
    experts = np.unique(ids)
    remap = np.full(d["E"], -1, np.int32)
    remap[experts] = np.arange(len(experts), dtype=np.int32)
    sel = torch.as_tensor(experts, device=d["w13"].device, dtype=torch.long)
    w13 = inputs.to_numpy_bits(d["w13"].index_select(0, sel))
    s13 = d["w13_scale"].index_select(0, sel).cpu().numpy()
    return oracle.h_scale(inputs.to_numpy_bits(d["x"]), w13, remap[ids], s13)


# Bound on the GPU's error in an E4M3 gate or up sum, relative to the sum of
# the magnitudes of its terms.  Measured on the 128-row E4M3 gate/up kernel
# (500-element sums): at most 6.2e-6 = 2^-17.3 of sum|t|, more than fp32
# accumulation alone would give, so the E4M3 MFMA's own accumulation is
# coarser than fp32; 2^-16 is the bound taken.
GATE_UP_EPS = 2.0 ** -16

# E4M3FN magnitudes of the 127 non-negative finite codes, ascending.
_E4M3_MAG = None


def _e4m3_mags():
    global _E4M3_MAG
    if _E4M3_MAG is None:
        _E4M3_MAG = np.array([oracle.e4m3_to_f64(c) for c in range(0x7F)], np.float64)
    return _E4M3_MAG


def flip_allowance(d, tokens, s_h, delta_s=0.0):
    """Per sampled token, the most its output row can move because E4M3 codes
    of h are decided on the far side of a rounding midpoint.  Encoding is a
    step function: where h / s_h lies within the GPU's error of the midpoint
    between two codes, either code is a correct rounding of a value that is
    itself correct within that error.  For each h element of the token's
    pairs (fp64, from the oracle's dequantised operands) the window is
    GATE_UP_EPS * (|dh/dg| S_g + |dh/du| S_u) + 2^-22 |h| (SiLU and scale
    roundings), plus delta_s * |h| for a scale that differs by delta_s; an
    element whose window holds a midpoint may take either neighbouring code,
    which moves out[t, n] by at most w_j * |w2[e, n, i]| * gap * s_h.
    Returns the absolute allowances [len(tokens), H]."""
    mags = _e4m3_mags()
    mids = (mags[1:] + mags[:-1]) / 2.0
    ids, wts = oracle.route_topk(d["logits"].cpu().numpy(), d["topk"], True)
    ids_t = ids[tokens]
    experts = np.unique(ids_t)
    sel = torch.as_tensor(experts, device=d["w13"].device, dtype=torch.long)
    table = np.array([oracle.e4m3_to_f64(c) for c in range(256)], np.float64)
    s13 = d["w13_scale"].index_select(0, sel).cpu().numpy().astype(np.float64)
    s2 = d["w2_scale"].index_select(0, sel).cpu().numpy().astype(np.float64)
    w13 = inputs.to_numpy_bits(d["w13"].index_select(0, sel))
    w2 = inputs.to_numpy_bits(d["w2"].index_select(0, sel))
    xb = inputs.to_numpy_bits(d["x"])
    sx = np.float32(oracle.act_scale(xb))
    xh = table[oracle.quantize_e4m3(xb[tokens], float(sx))] * np.float64(sx)
    I = w13.shape[1] // 2
    allow = np.zeros((len(tokens), w2.shape[1]))
    for c, e in enumerate(experts):
        rows, slots = np.nonzero(ids_t == e)
        W = table[w13[c]] * s13[c]
        g = xh[rows] @ W[:I].T
        u = xh[rows] @ W[I:].T
        Sg = np.abs(xh[rows]) @ np.abs(W[:I]).T
        Su = np.abs(xh[rows]) @ np.abs(W[I:]).T
        sg = 1.0 / (1.0 + np.exp(-g))
        h = g * sg * u
        dh_dg = np.abs(sg * (1.0 + g * (1.0 - sg)) * u)
        win = (GATE_UP_EPS * (dh_dg * Sg + np.abs(g * sg) * Su) + (2.0 ** -22 + delta_s) * np.abs(h)) / s_h
        q = np.minimum(np.abs(h) / s_h, 448.0)
        m = np.searchsorted(mids, q)  # nearest midpoints: mids[m - 1] <= q < mids[m]
        lo = np.clip(m - 1, 0, len(mids) - 1)
        hi = np.clip(m, 0, len(mids) - 1)
        near_lo = np.abs(q - mids[lo]) <= win
        near_hi = np.abs(q - mids[hi]) <= win
        gap = np.where(near_hi, mags[np.minimum(hi + 1, len(mags) - 1)] - mags[hi],
                       np.where(near_lo, mags[lo + 1] - mags[lo], 0.0))
        W2a = np.abs(table[w2[c]]) * s2[c]  # [H, I]
        a = (gap * s_h * wts[tokens[rows], slots][:, None]) @ W2a.T  # [rows, H]
        np.add.at(allow, rows, a)
    return allow


def row_err_with_allowance(got, ref, allow, tol):
    """max over rows of max_n (|g - r| - allow)+ / max|r|, to compare with tol."""
    num = np.maximum(np.abs(np.asarray(got, np.float64) - ref) - allow, 0.0).max(axis=1)
    den = np.abs(ref).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if len(num) else 0.0


def check_fp8_dynamic(d, scales, out, tokens, label, tol_own=FP8_TOL):
    """FP8 with the dynamic h scale.  (1) s_x bit-exact and s_h within
    SH_REL_TOL of the oracle's all-pairs scales; (2) the sampled rows against
    the oracle run at the GPU's s_h (the kernels' arithmetic, FP8_TOL);
    (3) the same rows against the oracle at its own s_h (the whole dynamic
    reading, tol_own).  scales: the device (s_x, s_h) pair the forward left
    in its workspace.  Returns (rel s_h difference, err at GPU s_h, err at
    oracle s_h)."""
    s_gpu = scales.cpu().numpy().astype(np.float64)
    ids, _ = oracle.route_topk(d["logits"].cpu().numpy(), d["topk"], True)
    sx_o, sh_o = oracle_h_scale(d, ids)
    assert s_gpu[0] == sx_o, (s_gpu[0], sx_o)
    rel = abs(s_gpu[1] / sh_o - 1.0)
    got = to_f64(out)[tokens]
    ref_g, _, _, _ = oracle_forward(d, tokens=tokens, a2_scale=float(s_gpu[1]))
    ref_o, _, _, _ = oracle_forward(d, tokens=tokens, a2_scale=sh_o)
    err_g = row_rel_err(got, ref_g)
    err_o = row_rel_err(got, ref_o)
    say(f"  {label}: s_h gpu {s_gpu[1]:.9g} oracle {sh_o:.9g} (rel {rel:.2e}); "
        f"rows {len(tokens)}: err at gpu s_h {err_g:.3e}, at oracle s_h {err_o:.3e}")
    assert rel <= SH_REL_TOL, rel
    if err_g > FP8_TOL or err_o > tol_own:
        # rows past the bar must be explained by codes decided at a midpoint
        ag = flip_allowance(d, tokens, float(s_gpu[1]))
        ao = flip_allowance(d, tokens, sh_o, delta_s=rel)
        eg = row_err_with_allowance(got, ref_g, ag, FP8_TOL)
        eo = row_err_with_allowance(got, ref_o, ao, tol_own)
        say(f"    beyond the codes decided within the GPU's error of a midpoint: "
            f"{eg:.3e} at gpu s_h, {eo:.3e} at oracle s_h")
        assert eg <= FP8_TOL, eg
        assert eo <= tol_own, eo
    return rel, err_g, err_o
