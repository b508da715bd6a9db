"""ctypes binding of oracle/libmoe_oracle.so (fp64 CPU oracle; test infrastructure).

Only tests/, the smoke check and the CPU-baseline leg of the benchmark use
this module.  Every function takes and returns numpy arrays.  Dtype codes:
0 = f32, 1 = bf16 (raw uint16 bits), 2 = E4M3FN (raw uint8 codes).  The
arithmetic lives in moe_oracle.c; this file marshals arguments, except
h_scale(), which forms the all-pairs h scale with fp64 library matrix
products so that it stays affordable at full batch sizes.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, E4M3 = 0, 1, 2

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        c_i64, c_i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_f64.restype = ctypes.c_double
        L.oracle_e4m3_from_f32.argtypes = [ctypes.c_float]
        L.oracle_e4m3_from_f32.restype = ctypes.c_uint8
        L.oracle_route_topk.argtypes = [vp, c_i64, c_i32, c_i32, c_i32, vp, vp]
        L.oracle_route_topk.restype = ctypes.c_int
        L.oracle_route_project.argtypes = [c_i32, vp, c_i32, vp, c_i64, c_i32, c_i32, c_i32,
                                           c_i32, vp, vp, vp]
        L.oracle_route_project.restype = ctypes.c_int
        L.oracle_align.argtypes = [vp, c_i64, c_i32, c_i32, c_i32, vp, vp, vp, vp, vp]
        L.oracle_align.restype = ctypes.c_int
        L.oracle_act_scale.argtypes = [c_i32, vp, c_i64]
        L.oracle_act_scale.restype = ctypes.c_float
        L.oracle_quantize_e4m3.argtypes = [c_i32, vp, c_i64, ctypes.c_float, vp]
        L.oracle_quantize_e4m3.restype = None
        L.oracle_moe_forward.argtypes = [c_i64, c_i32, c_i32, c_i32, c_i32,
                                         c_i32, vp, c_i32, vp, vp, vp, vp,
                                         c_i32, vp, vp, vp, vp, vp, c_i64, vp, vp]
        L.oracle_moe_forward.restype = ctypes.c_int
        L.oracle_rope_quant_per_head.argtypes = [c_i32, vp, vp, vp, c_i64, c_i32, c_i32, c_i32,
                                                 c_i32, vp, vp, vp, vp]
        L.oracle_rope_quant_per_head.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3
    raise TypeError(f"unsupported array dtype {a.dtype}")


def bf16_to_f64(bits):
    return lib().oracle_bf16_to_f64(int(bits))


def e4m3_to_f64(code):
    return lib().oracle_e4m3_to_f64(int(code))


def e4m3_from_f32(v):
    return int(lib().oracle_e4m3_from_f32(float(v)))


def route_topk(logits, topk, renormalize=True):
    """logits f32 [T,E] -> (ids int32 [T,k], weights f64 [T,k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.zeros((T, topk), np.int32)
    w = np.zeros((T, topk), np.float64)
    rc = lib().oracle_route_topk(_p(logits), T, E, topk, int(bool(renormalize)), _p(ids), _p(w))
    if rc:
        raise ValueError(f"oracle_route_topk failed ({rc})")
    return ids, w


def route_project(x, wr, topk, renormalize=True):
    """Linear router then top-k: x [T,K] and wr [E,K] (f32, or bf16 as uint16
    bits) -> (logits f64 [T,E], ids int32 [T,k], weights f64 [T,k])."""
    x = np.ascontiguousarray(x)
    wr = np.ascontiguousarray(wr)
    T, K = x.shape
    E, K2 = wr.shape
    if K2 != K:
        raise ValueError("x and wr disagree on K")
    logits = np.zeros((T, E), np.float64)
    ids = np.zeros((T, topk), np.int32)
    w = np.zeros((T, topk), np.float64)
    rc = lib().oracle_route_project(_dtype_code(x), _p(x), _dtype_code(wr), _p(wr), T, K, E, topk,
                                    int(bool(renormalize)), _p(logits), _p(ids), _p(w))
    if rc:
        raise ValueError(f"oracle_route_project failed ({rc})")
    return logits, ids, w


def align_capacity(T, topk, E, block_m):
    P = T * topk
    return P + min(E, P) * (block_m - 1)


def align(ids, E, block_m):
    """ids int32 [T,k] -> dict of the alignment arrays (defined ranges only)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    cap = max(align_capacity(T, k, E, block_m), 1)
    sorted_ids = np.full(cap, -7, np.int32)
    blocks = np.full((cap + block_m - 1) // block_m, -7, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    pair_pos = np.zeros(max(T * k, 1), np.int32)
    npad = np.zeros(1, np.int32)
    rc = lib().oracle_align(_p(ids), T, k, E, block_m, _p(sorted_ids), _p(blocks),
                            _p(offsets), _p(pair_pos), _p(npad))
    if rc:
        raise ValueError(f"oracle_align failed ({rc})")
    n = int(npad[0])
    return {"sorted_pair_ids": sorted_ids[:n].copy(),
            "block_expert_ids": blocks[: n // block_m].copy(),
            "expert_offsets": offsets, "pair_pos": pair_pos[: T * k].copy(),
            "num_padded": n}


def act_scale(x):
    x = np.ascontiguousarray(x)
    return float(lib().oracle_act_scale(_dtype_code(x), _p(x), x.size))


def quantize_e4m3(x, scale):
    x = np.ascontiguousarray(x)
    q = np.zeros(x.shape, np.uint8)
    lib().oracle_quantize_e4m3(_dtype_code(x), _p(x), x.size, float(scale), _p(q))
    return q


def moe_forward(x, w13, w2, ids, weights, w13_scale=None, w2_scale=None,
                fp8_act=False, a1_scale=None, a2_scale=None, tokens=None):
    """Reference fused MoE output in fp64.

    x: [T,H] float32 or uint16 (bf16 bits).  w13: [E,2I,H], w2: [E,H,I]
    (float32, uint16 bf16 bits or uint8 E4M3 codes).  ids/weights: [T,k].
    tokens: optional int64 list of rows to evaluate.  Returns (out f64
    [n,H], (s_x, s_h)).
    """
    x = np.ascontiguousarray(x)
    w13 = np.ascontiguousarray(w13)
    w2 = np.ascontiguousarray(w2)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    weights = np.ascontiguousarray(weights, dtype=np.float64)
    T, H = x.shape
    E, I2, H2 = w13.shape
    I = I2 // 2
    assert H2 == H and w2.shape == (E, H, I), (w13.shape, w2.shape)
    k = ids.shape[1]
    if tokens is not None:
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        n = tokens.size
    else:
        n = T
    out = np.zeros((max(n, 1), H), np.float64)
    scales = np.zeros(2, np.float32)
    s13 = None if w13_scale is None else np.ascontiguousarray(w13_scale, dtype=np.float32)
    s2 = None if w2_scale is None else np.ascontiguousarray(w2_scale, dtype=np.float32)
    a1 = None if a1_scale is None else np.array([a1_scale], np.float32)
    a2 = None if a2_scale is None else np.array([a2_scale], np.float32)
    rc = lib().oracle_moe_forward(T, H, I, E, k, _dtype_code(x), _p(x), _dtype_code(w13),
                                  _p(w13), _p(w2), _p(s13), _p(s2), int(bool(fp8_act)),
                                  _p(a1), _p(a2), _p(ids), _p(weights), _p(tokens), n,
                                  _p(out), _p(scales))
    if rc:
        raise ValueError(f"oracle_moe_forward failed ({rc})")
    return out[:n], (float(scales[0]), float(scales[1]))


def h_scale(x, w13, ids, w13_scale, a1_scale=None):
    """Dynamic per-tensor scale of the FP8 intermediate over every real pair
    of the batch (the per-tensor scaling of the AWS post, "Backend routing for
    FP8 tensor quantization", read as for x): s_h = fl32(amax|h| / 448), with
    h = SiLU(g) * u, g and u the gate and up projections of the dequantised
    activations x^ = s_x * E4M3(fl32(x / s_x)) by s13[e] * w13[e].

    Same definition as the dynamic path of moe_forward; here each expert's
    gate/up product over all of its tokens is one fp64 library matmul
    (numpy), which only changes the order of the fp64 sums.  x: [T,H] f32 or
    bf16 bits; w13: [E,2I,H] E4M3 codes; ids: [T,k] (ids index w13's first
    axis); w13_scale: [E] f32.  Returns (s_x, s_h) as Python floats."""
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, H = x.shape
    E, I2, H2 = w13.shape
    assert H2 == H and w13.dtype == np.uint8
    I = I2 // 2
    k = ids.shape[1]
    sx = np.float32(a1_scale) if a1_scale is not None else np.float32(act_scale(x))
    table = np.array([e4m3_to_f64(c) for c in range(256)], np.float64)
    xh = table[quantize_e4m3(x, float(sx))] * np.float64(sx)
    flat = ids.reshape(-1)
    amax = 0.0
    for e in np.unique(flat):
        rows = np.nonzero(flat == e)[0] // k  # a token lists an expert at most once
        W = table[w13[e]] * np.float64(np.float32(w13_scale[e]))
        xe = xh[rows]
        g = xe @ W[:I].T
        u = xe @ W[I:].T
        h = g / (1.0 + np.exp(-g)) * u
        amax = max(amax, float(np.abs(h).max()))
    sh = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    return float(sx), float(sh)


def rope_quant_per_head(x, positions, inv_freq, interleaved=False, inverse=False,
                        static_scales=None, want_y=False):
    """Rotary embedding then per-head E4M3 codes (moe_oracle.c,
    oracle_rope_quant_per_head).  x: [T, nH, D] float32 or uint16 (bf16
    bits); positions: [T] int32; inv_freq: [D/2] float32.  Returns (codes
    uint8 [T, nH, D], scales f32 [nH]) and, with want_y, the fp64 rotated
    values."""
    x = np.ascontiguousarray(x)
    T, nH, D = x.shape
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    invf = np.ascontiguousarray(inv_freq, dtype=np.float32)
    assert pos.shape == (T,) and invf.shape == (D // 2,)
    codes = np.zeros((T, nH, D), np.uint8)
    scales = np.zeros(nH, np.float32)
    y = np.zeros((T, nH, D), np.float64) if want_y else None
    st = None if static_scales is None else np.ascontiguousarray(static_scales, dtype=np.float32)
    rc = lib().oracle_rope_quant_per_head(_dtype_code(x), _p(x), _p(pos), _p(invf), T, nH, D,
                                          int(bool(interleaved)), int(bool(inverse)), _p(st),
                                          _p(codes), _p(scales), _p(y))
    if rc:
        raise ValueError(f"oracle_rope_quant_per_head failed ({rc})")
    return (codes, scales, y) if want_y else (codes, scales)
