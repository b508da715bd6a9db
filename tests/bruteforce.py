"""Independent brute-force checks used to pin the oracle (CPU only).

Nothing here shares code with oracle/ or with the GPU library.  Decoding of
bf16 and E4M3 goes through torch's own dtypes (library routines); products go
through numpy matmul in fp64; routing uses a full lexicographic sort; the
alignment uses Python's sorted().
"""
import numpy as np
import torch


def decode(a):
    """numpy array of raw bits (float32 / uint16 bf16 / uint8 E4M3) -> fp64."""
    if a.dtype == np.float32:
        return a.astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        return t.view(torch.bfloat16).to(torch.float64).numpy()
    if a.dtype == np.uint8:
        return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    raise TypeError(a.dtype)


def e4m3_cast(v32):
    """fp32 -> nearest E4M3FN (ties to even) via torch's cast, saturated first."""
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def route(logits, k, renormalize=True):
    logits = np.asarray(logits, np.float32)
    T, E = logits.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        sel = order[:k]
        l64 = logits[t].astype(np.float64)
        p = np.exp(l64 - l64.max())
        p = p / p.sum()
        ids[t] = sel
        w[t] = p[sel] / p[sel].sum() if renormalize else p[sel]
    return ids, w


def align(ids, E, bm):
    ids = np.asarray(ids)
    T, k = ids.shape
    P = T * k
    flat = ids.reshape(-1)
    order = sorted(range(P), key=lambda f: (int(flat[f]), f))
    sorted_ids, blocks, offsets = [], [], []
    pos = {}
    i = 0
    for e in range(E):
        offsets.append(len(sorted_ids))
        members = []
        while i < P and flat[order[i]] == e:
            members.append(order[i])
            i += 1
        padded = -(-len(members) // bm) * bm
        for f in members:
            pos[f] = len(sorted_ids)
            sorted_ids.append(f)
        sorted_ids.extend([P] * (padded - len(members)))
        blocks.extend([e] * (padded // bm))
    offsets.append(len(sorted_ids))
    return {"sorted_pair_ids": np.array(sorted_ids, np.int32),
            "block_expert_ids": np.array(blocks, np.int32),
            "expert_offsets": np.array(offsets, np.int32),
            "pair_pos": np.array([pos[f] for f in range(P)], np.int32),
            "num_padded": len(sorted_ids)}


def silu(z):
    return z / (1.0 + np.exp(-z))


def expert_ffn_all(x, w13, w2):
    """FFN_e(x) for every expert and every row: [E, T, H] via matmul."""
    E, I2, H = w13.shape
    I = I2 // 2
    out = []
    for e in range(E):
        g = x @ w13[e, :I].T
        u = x @ w13[e, I:].T
        out.append((silu(g) * u) @ w2[e].T)
    return np.stack(out)


def dense_gated(x, w13, w2, ids, w):
    """out[t] = sum_e G[t,e] FFN_e(x_t), G zero outside each token's top-k."""
    T = x.shape[0]
    E = w13.shape[0]
    G = np.zeros((T, E))
    for t in range(T):
        for j in range(ids.shape[1]):
            G[t, ids[t, j]] += w[t, j]
    y = expert_ffn_all(x, w13, w2)
    return np.einsum("te,eth->th", G, y)


def fp8_forward(x_bits, w13q, w2q, s13, s2, ids, w):
    """FP8 path written with torch's E4M3 cast and numpy matmul:
    x: one dynamic scale amax/448 (fp32), codes of fl32(x / s);
    h: one dynamic scale fl32(amax/448) over all real pairs (amax of the fp64
    values), codes of fl32(h / s_h) with the quotient formed in fp64."""
    x32 = decode(x_bits).astype(np.float32)
    amax = np.float32(np.abs(x32).max())
    sx = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    xd = e4m3_cast(x32 / sx) * np.float64(sx)
    w13d = decode(w13q) * s13.astype(np.float64)[:, None, None]
    w2d = decode(w2q) * s2.astype(np.float64)[:, None, None]
    T, k = ids.shape
    I = w13d.shape[1] // 2
    hs = np.zeros((T, k, I))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            hs[t, j] = silu(w13d[e, :I] @ xd[t]) * (w13d[e, I:] @ xd[t])
    hmax = np.abs(hs).max()
    sh = np.float32(hmax / 448.0) if hmax > 0 else np.float32(1.0)
    hq = e4m3_cast((hs / np.float64(sh)).astype(np.float32)) * np.float64(sh)
    out = np.zeros((T, w2d.shape[1]))
    for t in range(T):
        for j in range(k):
            out[t] += w[t, j] * (w2d[ids[t, j]] @ hq[t, j])
    return out, float(sx), float(sh)
