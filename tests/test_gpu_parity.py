"""Parity of the HIP path (called through the C ABI) with the fp64 oracle.

Bars: routing ids, the alignment and the E4M3 codes of x bit-exact; routing
weights within 1e-6 relative; outputs within a per-row relative error of 1e-2
(f32/bf16 weights) or 3e-2 (E4M3 weights).  Small shapes span several tiles
and ragged tails of both kernel families; the full workload sizes are checked
on sampled tokens.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_13_amd import inputs, moe
from tests import bruteforce as bf
from tests import harness as H

pytestmark = pytest.mark.gpu

DEV = "cuda"
W = inputs.WORKLOADS


@pytest.fixture(autouse=True)
def _announce(request):
    H.say(f"\n[gpu-test] {request.node.name}")
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ routing

ROUTE_CASES = [(16, 8, 2, 0.0), (1, 64, 8, 0.0), (64, 64, 8, 0.0), (256, 256, 8, 1.1),
               (8192, 64, 8, 1.1), (5, 1024, 64, 0.0), (37, 1000, 17, 0.0), (3, 2, 1, 0.0)]


@pytest.mark.parametrize("T,E,k,zipf", ROUTE_CASES)
@pytest.mark.parametrize("renorm", [True, False])
def test_route_topk_matches_oracle(T, E, k, zipf, renorm):
    logits = inputs.make_logits(T, E, 77 + T + E, zipf, device=DEV)
    ids, w = moe.moe_route_topk(logits, k, renorm)
    torch.cuda.synchronize()
    rids, rw = oracle.route_topk(logits.cpu().numpy(), k, renorm)
    assert np.array_equal(ids.cpu().numpy(), rids)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6, atol=1e-7)


# Router projection fused with the routing (logits = x . W_r^T).  The GPU
# selects on its fp32 logits: (1) those logits match the fp64 projection
# within the bound of the arithmetic (bf16 products are exact in fp32, so
# only the fp32 sum errs: K * 2^-24 * sum|x w|, taken 2^-20 * sum|x w| + 1e-6;
# f32 inputs are rounded to bf16 first: 2^-8 relative per product); (2) the
# ids and weights are exactly the routing of those fp32 logits (the pinned
# routing oracle on the GPU's own logits); (3) against the fp64 router the
# ids are identical wherever the k-th boundary is clear of that bound, and
# elsewhere still a valid top-k.
ROUTER_CASES = [
    # name, T, K, E, k, dtype
    ("bf16_T1_E64", 1, 4096, 64, 8, torch.bfloat16),
    ("bf16_T64_E64", 64, 4096, 64, 8, torch.bfloat16),
    ("bf16_T37_E256", 37, 7168, 256, 8, torch.bfloat16),
    ("bf16_T20_E8_ksplit16", 20, 256, 8, 2, torch.bfloat16),
    ("f32_T16_E8", 16, 256, 8, 2, torch.float32),
    ("bf16_T5_E1000", 5, 512, 1000, 17, torch.bfloat16),
    ("bf16_T130_E48_ksplit5", 130, 1024, 48, 6, torch.bfloat16),
    ("bf16_T300_E64", 300, 4096, 64, 8, torch.bfloat16),
    # 64 token blocks: 16 K slices of 256, two K steps per projection wave
    ("bf16_T4096_E64_multistep", 4096, 4096, 64, 8, torch.bfloat16),
]


def _bits(t):
    t = t.cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


@pytest.mark.parametrize("name,T,K,E,k,dt", ROUTER_CASES, ids=[c[0] for c in ROUTER_CASES])
@pytest.mark.parametrize("renorm", [True, False])
def test_route_project_matches_oracle(name, T, K, E, k, dt, renorm):
    x = inputs.make_x(T, K, 500 + T, dt, device=DEV)
    wr = inputs.make_router(E, K, 600 + E, dt, device=DEV)
    logits = torch.empty(T, E, dtype=torch.float32, device=DEV)
    ids, w = moe.moe_route_project_topk(x, wr, k, renorm, logits=logits)
    torch.cuda.synchronize()
    gl = logits.cpu().numpy()
    l64, oids, _ = oracle.route_project(_bits(x), _bits(wr), k, renorm)
    xa = np.abs(bf.decode(_bits(x)))
    wa = np.abs(bf.decode(_bits(wr)))
    S = xa @ wa.T  # sum_k |x w| per (t, e)
    bound = (2.0 ** -8 * 3 if dt == torch.float32 else 2.0 ** -20) * S + 1e-6
    assert np.all(np.abs(gl.astype(np.float64) - l64) <= bound), np.max(np.abs(gl - l64) / bound)
    # ids and weights are the routing of the GPU's own logits
    rids, rw = oracle.route_topk(gl, k, renorm)
    gids = ids.cpu().numpy()
    assert np.array_equal(gids, rids)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    # against the fp64 router: exact where the boundary is clear, else valid
    delta = 2 * bound.max(axis=1)
    srt = -np.sort(-l64, axis=1)
    lk = srt[:, k - 1]
    nxt = srt[:, k] if k < E else np.full(T, -np.inf)
    clear = (lk - nxt) > delta
    gaps = np.min(srt[:, :k - 1] - srt[:, 1:k], axis=1) if k > 1 else np.full(T, np.inf)
    clear_order = clear & (gaps > delta)
    assert np.array_equal(gids[clear_order], oids[clear_order])
    assert np.array_equal(np.sort(gids[clear], 1), np.sort(oids[clear], 1))
    for t in np.nonzero(~clear)[0]:
        sel = l64[t, gids[t]]
        assert len(set(gids[t].tolist())) == k and np.all(sel >= lk[t] - delta[t])
    H.say(f"  {name}: max |dlogit| {np.max(np.abs(gl - l64)):.2e}, rows with a near tie {int((~clear_order).sum())}/{T}")


def test_route_project_logits_optional_and_empty():
    x = inputs.make_x(24, 512, 7, torch.bfloat16, device=DEV)
    wr = inputs.make_router(64, 512, 8, torch.bfloat16, device=DEV)
    lg = torch.empty(24, 64, dtype=torch.float32, device=DEV)
    i1, w1 = moe.moe_route_project_topk(x, wr, 8, logits=lg)
    i2, w2 = moe.moe_route_project_topk(x, wr, 8)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(w1, w2)
    e = torch.empty(0, 512, dtype=torch.bfloat16, device=DEV)
    ie, we = moe.moe_route_project_topk(e, wr, 8)
    assert ie.shape == (0, 8) and we.shape == (0, 8)


def test_route_ties_go_to_lower_id():
    l = torch.zeros(4, 64, device=DEV)
    l[1] = -0.0
    l[2, ::3] = -0.0
    l[3, 10:20] = 1.5
    ids, w = moe.moe_route_topk(l, 8, True)
    torch.cuda.synchronize()
    rids, rw = oracle.route_topk(l.cpu().numpy(), 8, True)
    assert np.array_equal(ids.cpu().numpy(), rids)
    assert list(rids[0]) == list(range(8)) and list(rids[3]) == list(range(10, 18))
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6)


def test_route_empty_batch():
    ids, w = moe.moe_route_topk(torch.zeros(0, 64, device=DEV), 8)
    assert ids.shape == (0, 8)


# ---------------------------------------------------------------- alignment

ALIGN_CASES = [(1, 64, 8), (16, 8, 2), (64, 64, 8), (129, 8, 8), (256, 256, 8),
               (300, 1024, 4), (8192, 64, 8)]


@pytest.mark.parametrize("bm", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("T,E,k", ALIGN_CASES)
def test_align_matches_oracle(T, E, k, bm):
    logits = inputs.make_logits(T, E, 5 + T, 1.1 if E > 8 else 0.0, device=DEV)
    ids, _ = moe.moe_route_topk(logits, k)
    p = moe.make_problem(T, 128, 128, E, k, bm, torch.bfloat16, torch.bfloat16, torch.bfloat16)
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device=DEV)
    al = moe.moe_align_permute(ids, E, bm, ws)
    torch.cuda.synchronize()
    ref = oracle.align(ids.cpu().numpy(), E, bm)
    n = int(al.num_padded.item())
    assert n == ref["num_padded"]
    assert np.array_equal(al.expert_offsets.cpu().numpy(), ref["expert_offsets"])
    assert np.array_equal(al.sorted_pair_ids[:n].cpu().numpy(), ref["sorted_pair_ids"])
    assert np.array_equal(al.block_expert_ids[: n // bm].cpu().numpy(), ref["block_expert_ids"])
    assert np.array_equal(al.pair_pos[: T * k].cpu().numpy(), ref["pair_pos"])


def test_align_drops_out_of_range_ids():
    ids = torch.tensor([[0, 3], [7, -1], [8, 3], [2, 2]], dtype=torch.int32, device=DEV)
    al = moe.moe_align_permute(ids, 8, 16, torch.empty(16, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    ref = oracle.align(ids.cpu().numpy(), 8, 16)
    n = int(al.num_padded.item())
    assert n == ref["num_padded"]
    assert np.array_equal(al.sorted_pair_ids[:n].cpu().numpy(), ref["sorted_pair_ids"])
    assert np.array_equal(al.pair_pos[:8].cpu().numpy(), ref["pair_pos"])
    assert ref["pair_pos"][3] == -1 and ref["pair_pos"][4] == -1


def test_align_empty_batch():
    ids = torch.zeros(0, 8, dtype=torch.int32, device=DEV)
    al = moe.moe_align_permute(ids, 64, 16, torch.empty(16, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert int(al.num_padded.item()) == 0
    assert int(al.expert_offsets.abs().sum().item()) == 0


def test_align_is_deterministic():
    logits = inputs.make_logits(8192, 64, 3, 1.1, device=DEV)
    ids, _ = moe.moe_route_topk(logits, 8)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    a = moe.moe_align_permute(ids, 64, 128, ws)
    s1 = a.sorted_pair_ids.clone()
    b = moe.moe_align_permute(ids, 64, 128, ws)
    n = int(a.num_padded.item())
    assert torch.equal(s1[:n], b.sorted_pair_ids[:n])


@pytest.mark.parametrize("T,E,k,bm", [(1, 64, 8, 16), (8, 64, 8, 16), (64, 64, 8, 16), (16, 8, 2, 32), (37, 1000, 17, 64),
                                       (128, 256, 8, 16), (129, 64, 8, 128), (3, 2, 1, 16)])
def test_route_align_fused_equals_separate_calls(T, E, k, bm):
    logits = inputs.make_logits(T, E, 31 + T, 1.1 if E > 8 else 0.0, device=DEV)
    p = moe.make_problem(max(T, 1), 128, 128, E, k, bm, torch.bfloat16, torch.bfloat16, torch.bfloat16)
    ws = torch.empty(moe.moe_workspace_size(p), dtype=torch.uint8, device=DEV)
    ids_a, w_a = moe.moe_route_topk(logits, k, True)
    al_a = moe.moe_align_permute(ids_a, E, bm, ws)
    torch.cuda.synchronize()
    ids_b, w_b, al_b = moe.moe_route_align(logits, k, True, bm, ws)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b) and torch.equal(w_a, w_b)
    n = int(al_a.num_padded.item())
    assert n == int(al_b.num_padded.item())
    assert torch.equal(al_a.expert_offsets, al_b.expert_offsets)
    assert torch.equal(al_a.sorted_pair_ids[:n], al_b.sorted_pair_ids[:n])
    assert torch.equal(al_a.block_expert_ids[: n // bm], al_b.block_expert_ids[: n // bm])
    assert torch.equal(al_a.pair_pos[: T * k], al_b.pair_pos[: T * k])
    ref = oracle.align(oracle.route_topk(logits.cpu().numpy(), k, True)[0], E, bm)
    assert np.array_equal(al_b.sorted_pair_ids[:n].cpu().numpy(), ref["sorted_pair_ids"])


# ------------------------------------------------------- activation quant

@pytest.mark.parametrize("shape,dtype", [((1, 4096), torch.bfloat16), ((64, 4096), torch.bfloat16),
                                         ((16, 256), torch.float32), ((256, 7168), torch.bfloat16),
                                         ((333, 384), torch.float32)])
def test_quantize_act_codes_bit_exact(shape, dtype):
    x = inputs.make_x(shape[0], shape[1], 9 + shape[0], dtype, 1.0, device=DEV)
    x[0, :5] = torch.tensor([0.0, -0.0, 1e-6, -3e-3, 2.0], dtype=dtype)
    codes, s = moe.moe_quantize_act(x)
    torch.cuda.synchronize()
    xb = inputs.to_numpy_bits(x)
    rs = oracle.act_scale(xb)
    assert float(s.item()) == rs
    ref = oracle.quantize_e4m3(xb, rs)
    assert np.array_equal(codes.cpu().numpy(), ref)


def test_quantize_act_static_scale_and_zero_input():
    x = inputs.make_x(64, 1024, 1, torch.bfloat16, 3.0, device=DEV)
    st = torch.tensor([0.01], device=DEV)
    codes, s = moe.moe_quantize_act(x, static_scale=st)
    torch.cuda.synchronize()
    assert float(s.item()) == np.float32(0.01)
    ref = oracle.quantize_e4m3(inputs.to_numpy_bits(x), float(np.float32(0.01)))
    assert np.array_equal(codes.cpu().numpy(), ref)  # includes saturated codes
    z = torch.zeros(8, 256, dtype=torch.bfloat16, device=DEV)
    codes, s = moe.moe_quantize_act(z)
    torch.cuda.synchronize()
    assert float(s.item()) == 1.0 and int(codes.sum().item()) == 0


# --------------------------------------------------------- forward (small)

SMALL = [
    # name, workload, T, H, I, E, k, block_m
    ("tiny_fp32_full", "tiny_fp32", 16, None, None, None, None, 16),
    ("tiny_fp32_T1", "tiny_fp32", 1, None, None, None, None, 16),
    ("f32_tile", "tiny_fp32", 100, None, None, None, None, 32),
    ("bf16_T1", "decode_bf16", 1, 512, 256, 16, 4, 16),
    ("bf16_T7", "decode_bf16", 7, 512, 384, 16, 4, 16),
    ("bf16_T33", "decode_bf16", 33, 768, 256, 16, 4, 32),
    ("bf16_T64", "decode_bf16", 64, 512, 256, 8, 3, 64),
    ("bf16_T65_tile", "decode_bf16", 65, 512, 256, 16, 4, 16),
    ("bf16_T200_tile", "decode_bf16", 200, 640, 384, 12, 4, 128),
    ("bf16_T300_bm256", "decode_bf16", 300, 512, 256, 8, 2, 256),
    ("bf16_T5_K256", "decode_bf16", 5, 256, 128, 4, 2, 16),   # one 512-byte ring stage per row
    ("fp8_T9_K512_N512", "decode_fp8", 9, 512, 512, 8, 2, 16),  # both rings one stage per task
    # 16-row blocks with experts of 2-4 blocks: gate/up column groups of two
    # blocks of one expert, odd block counts, groups whose second block
    # belongs to the next expert (uniform and Zipf routing)
    ("bf16_T60_span", "decode_bf16", 60, 512, 256, 4, 2, 16),
    ("bf16_T48_span_zipf", "prefill_bf16", 48, 512, 384, 8, 4, 16),
    ("fp8_T50_span_zipf", "large_fp8", 50, 512, 256, 8, 4, 16),
    ("fp8_T1", "decode_fp8", 1, 512, 256, 16, 4, 16),
    # more than 32 Ki activations: the two-launch quantisation of x (partial
    # maxima, then s_x and the codes) ahead of the gate/up ring
    ("fp8_T40_K1024", "decode_fp8", 40, 1024, 256, 16, 4, 16),
    ("fp8_T19", "decode_fp8", 19, 1024, 256, 16, 4, 16),
    ("fp8_T64", "decode_fp8", 64, 512, 384, 16, 8, 32),
    ("fp8_T100_tile", "decode_fp8", 100, 512, 256, 16, 4, 64),
    ("fp8_T257_tile", "large_fp8", 257, 768, 256, 32, 8, 128),
    # degenerate routings: every expert for every token (k = E = 64, the
    # largest k; more than one alignment chunk of pairs at 20 tokens), and
    # top-1
    ("bf16_T20_k64_E64", "decode_bf16", 20, 512, 256, 64, 64, 16),
    ("fp8_T3_k64_E64", "decode_fp8", 3, 512, 256, 64, 64, 16),
    ("bf16_T50_k1", "decode_bf16", 50, 512, 256, 16, 1, 16),
]

# Large-batch kernels (alignment blocks of 128 or 256 rows): 1, 2, 3, 4 and 5
# chunks of K, ragged expert segments.  FP8 cases run the dynamic h scale (the
# layer's default): s_h is checked against the oracle's all-pairs scale, the
# rows against the oracle at the GPU's s_h (the kernels' arithmetic) and at
# its own s_h (the whole dynamic reading).
PREFILL_SMALL = [
    ("fp8_T150_I128", "decode_fp8", 150, 512, 128, 8, 4, 128),
    ("fp8_T140_I384", "decode_fp8", 140, 512, 384, 8, 4, 256),
    ("fp8_T130_K640", "decode_fp8", 130, 640, 384, 8, 2, 128),
    ("bf16_T129_I128", "decode_bf16", 129, 768, 128, 8, 4, 256),
    ("bf16_T520_E4", "decode_bf16", 520, 512, 256, 4, 2, 128),
    # persistent launches: runs of several tiles per workgroup, the DMA ring
    # carried across tile boundaries (8-16 chunks of K, 104 tiles)
    ("bf16_T600_persist", "decode_bf16", 600, 1024, 512, 8, 4, 128),
    ("fp8_T600_persist", "decode_fp8", 600, 1024, 512, 8, 4, 128),
    ("fp8_T700_persist_bm256", "large_fp8", 700, 1024, 512, 16, 4, 256),
    # 256 x 256 tiles (256-row blocks) for both products, bf16 and E4M3
    ("bf16_T900_bm256", "decode_bf16", 900, 1024, 512, 8, 4, 256),
    ("fp8_T900_bm256", "decode_fp8", 900, 1024, 1024, 8, 4, 256),
    ("fp8_T1100_I512_bm256", "prefill_fp8", 1100, 768, 512, 8, 4, 256),
]


@pytest.mark.parametrize("name,wl,T,Hd,Id,Ed,kd,bm", PREFILL_SMALL, ids=[c[0] for c in PREFILL_SMALL])
def test_forward_prefill_kernels_match_oracle(name, wl, T, Hd, Id, Ed, kd, bm):
    w = W[wl]
    d = inputs.make_inputs(w, T, device=DEV, H=Hd, I=Id, E=Ed, topk=kd)
    layer, out = H.run_gpu(d, block_m=bm)
    rids, _ = oracle.route_topk(d["logits"].cpu().numpy(), kd, True)
    assert np.array_equal(layer.topk_ids.cpu().numpy(), rids)
    if w.fp8_act:
        H.check_fp8_dynamic(d, layer.act_scales(), out, np.arange(T), name)
        return
    ref, _, _, _ = H.oracle_forward(d)
    err = H.row_rel_err(H.to_f64(out), ref)
    H.say(f"  {name}: max row rel err {err:.3e} (tol {H.BF16_TOL})")
    assert err <= H.BF16_TOL, err


@pytest.mark.parametrize("name,wl,T,Hd,Id,Ed,kd,bm", SMALL, ids=[c[0] for c in SMALL])
def test_forward_small_matches_oracle(name, wl, T, Hd, Id, Ed, kd, bm):
    w = W[wl]
    d = inputs.make_inputs(w, T, device=DEV, H=Hd, I=Id, E=Ed, topk=kd)
    layer, out = H.run_gpu(d, block_m=bm)
    ref, rids, _, (sx, sh) = H.oracle_forward(d)
    assert np.array_equal(layer.topk_ids.cpu().numpy(), rids)
    if w.fp8_act:
        H.check_fp8_dynamic(d, layer.act_scales(), out, np.arange(T), name)
    err = H.row_rel_err(H.to_f64(out), ref)
    tol = H.FP8_TOL if w.fp8_act else H.BF16_TOL
    H.say(f"  {name}: max row rel err {err:.3e} (tol {tol})")
    assert err <= tol, err


# Decode shapes whose gate/up task table does not fit beside two rings per
# CU (64 tokens, 1024 experts, 32-row alignment blocks: the capacity bound is
# 512 blocks x 64 row blocks = 32768 tasks, 65 per workgroup at 512
# workgroups, 9.4 KiB of table next to 65 KiB of ring and 12 KiB of partial
# sums), so the layer runs the one-workgroup-per-CU launch of the same kernel.
@pytest.mark.parametrize("wl", ["decode_bf16", "decode_fp8"])
def test_forward_gate_up_ring_one_workgroup_per_cu(wl):
    w = W[wl]
    d = inputs.make_inputs(w, 64, device=DEV, H=1024, I=1024, E=1024, topk=8)
    layer, out = H.run_gpu(d, block_m=32)
    tokens = np.arange(64)
    rids, _ = oracle.route_topk(d["logits"].cpu().numpy(), 8, True)
    assert np.array_equal(layer.topk_ids.cpu().numpy(), rids)
    if w.fp8_act:
        H.check_fp8_dynamic(d, layer.act_scales(), out, tokens, f"{wl} E=1024 bm=32")
        return
    ref, _, _, _ = H.oracle_forward(d, tokens=tokens)
    err = H.row_rel_err(H.to_f64(out)[tokens], ref)
    H.say(f"  {wl} E=1024 bm=32: max row rel err {err:.3e}")
    assert err <= H.BF16_TOL, err


def test_forward_fp8_static_scales():
    d = inputs.make_inputs(W["decode_fp8"], 24, device=DEV, H=512, I=256, E=16, topk=4)
    layer, out = H.run_gpu(d, a1_scale=0.02, a2_scale=0.01)
    ref, _, _, (sx, sh) = H.oracle_forward(d, a1_scale=0.02, a2_scale=0.01)
    assert (sx, sh) == (np.float32(0.02), np.float32(0.01))
    assert H.row_rel_err(H.to_f64(out), ref) <= H.FP8_TOL


def test_forward_not_renormalized():
    d = inputs.make_inputs(W["decode_bf16"], 9, device=DEV, H=512, I=256, E=16, topk=4)
    layer, out = H.run_gpu(d, renormalize=False)
    ref, _, _, _ = H.oracle_forward(d, renormalize=False)
    assert H.row_rel_err(H.to_f64(out), ref) <= H.BF16_TOL


def test_forward_f32_output():
    d = inputs.make_inputs(W["decode_bf16"], 5, device=DEV, H=512, I=256, E=16, topk=4)
    layer, out = H.run_gpu(d, out_dtype=torch.float32)
    assert out.dtype == torch.float32
    ref, _, _, _ = H.oracle_forward(d)
    assert H.row_rel_err(H.to_f64(out), ref) <= H.BF16_TOL


def test_forward_is_deterministic():
    for wl, T in (("decode_bf16", 33), ("decode_fp8", 150)):
        d = inputs.make_inputs(W[wl], T, device=DEV, H=512, I=256, E=16, topk=4)
        layer, out = H.run_gpu(d)
        first = out.clone()
        out2 = layer(d["x"], d["logits"])
        torch.cuda.synchronize()
        assert torch.equal(first, out2)


def test_graph_replay_matches_eager():
    d = inputs.make_inputs(W["decode_fp8"], 32, device=DEV, H=512, I=256, E=16, topk=4)
    layer, _ = H.run_gpu(d)
    x = d["x"].clone()
    logits = d["logits"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        layer(x, logits)  # warm on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            layer(x, logits)
    torch.cuda.synchronize()
    for rep in range(4):
        new = inputs.make_inputs(W["decode_fp8"], 32, device=DEV, seed=500 + rep, H=512, I=256,
                                 E=16, topk=4)
        x.copy_(new["x"])
        logits.copy_(new["logits"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = layer.out.clone()
        eager = layer(new["x"], new["logits"]).clone()
        torch.cuda.synchronize()
        assert torch.equal(got, eager), rep


# ------------------------------------------------ forward (full, sampled)

# Every workload at every size it names, at the layer's default alignment
# block (what the benchmark runs), on up to 256 tokens: all of them up to 256
# tokens, else the token of the last real pair of every expert segment plus a
# seeded random fill.  FP8 runs the dynamic h scale against the oracle's
# all-pairs scale.
FULL = [("decode_bf16", 1), ("decode_bf16", 8), ("decode_bf16", 32), ("decode_bf16", 64),
        ("decode_fp8", 1), ("decode_fp8", 8), ("decode_fp8", 32), ("decode_fp8", 64),
        ("large_fp8", 1), ("large_fp8", 16), ("large_fp8", 64), ("large_fp8", 256),
        ("prefill_bf16", 4096), ("prefill_bf16", 8192),
        ("prefill_fp8", 4096), ("prefill_fp8", 8192)]


@pytest.mark.parametrize("wl,T", FULL, ids=[f"{a}-T{b}" for a, b in FULL])
def test_forward_full_size_sampled_tokens(wl, T):
    w = W[wl]
    d = inputs.make_inputs(w, T, device=DEV)
    layer, out = H.run_gpu(d)
    rids, _ = oracle.route_topk(d["logits"].cpu().numpy(), d["topk"], True)
    assert np.array_equal(layer.topk_ids.cpu().numpy(), rids)
    tokens = H.sample_tokens(rids, 256, seed=T)
    label = f"{wl} T={T} block_m={layer.block_m}"
    if w.fp8_act:
        H.check_fp8_dynamic(d, layer.act_scales(), out, tokens, label)
    else:
        ref, _, _, _ = H.oracle_forward(d, tokens=tokens)
        err = H.row_rel_err(H.to_f64(out)[tokens], ref)
        H.say(f"  {label}: {len(tokens)} rows, max row rel err {err:.3e}")
        assert err <= H.BF16_TOL, err
    # whole-batch properties at full size: finite, no row left unwritten
    o = out.float()
    assert torch.isfinite(o).all()
    assert (o.abs().amax(dim=1) > 0).all()


# The same check on batches drawn from other seeds (new x, logits and
# weights): the routing and the per-tensor scales change with them, and so do
# the expert loads, padding and tile counts the kernels walk.
SEEDED = [(wl, T, sd) for wl, T in [("decode_bf16", 64), ("decode_fp8", 64), ("large_fp8", 64),
                                     ("large_fp8", 256), ("prefill_bf16", 8192), ("prefill_fp8", 8192)]
          for sd in (11, 3333)]


@pytest.mark.parametrize("wl,T,sd", SEEDED, ids=[f"{a}-T{b}-seed{c}" for a, b, c in SEEDED])
def test_forward_full_size_other_seeds(wl, T, sd):
    w = W[wl]
    d = inputs.make_inputs(w, T, device=DEV, seed=90000 + 7 * sd + T)
    layer, out = H.run_gpu(d)
    rids, _ = oracle.route_topk(d["logits"].cpu().numpy(), d["topk"], True)
    assert np.array_equal(layer.topk_ids.cpu().numpy(), rids)
    tokens = H.sample_tokens(rids, 128, seed=sd)
    label = f"{wl} T={T} seed {sd} block_m={layer.block_m}"
    if w.fp8_act:
        H.check_fp8_dynamic(d, layer.act_scales(), out, tokens, label)
    else:
        ref, _, _, _ = H.oracle_forward(d, tokens=tokens)
        err = H.row_rel_err(H.to_f64(out)[tokens], ref)
        H.say(f"  {label}: {len(tokens)} rows, max row rel err {err:.3e}")
        assert err <= H.BF16_TOL, err
    o = out.float()
    assert torch.isfinite(o).all()
    assert (o.abs().amax(dim=1) > 0).all()


# ------------------------------------------- pre-quantised activations

PREQUANT = [("decode_fp8", 1, {}), ("decode_fp8", 3, {}), ("decode_fp8", 8, {}),
            ("decode_fp8", 64, {}), ("large_fp8", 256, {}),
            ("prefill_fp8", 1100, dict(H=768, I=512, E=8, topk=4))]


@pytest.mark.parametrize("wl,T,shape", PREQUANT, ids=[f"{c[0]}_T{c[1]}" for c in PREQUANT])
def test_prequantised_activations_equal_internal_quantisation(wl, T, shape):
    """E4M3 codes made beforehand by moe_quantize_act and handed to
    moe_fused_forward with their scale give the same s_x, s_h and output,
    bit for bit, as the forward that quantises x itself (the same codes from
    the same kernels)."""
    w = W[wl]
    d = inputs.make_inputs(w, T, device=DEV, seed=300 + T, **shape)
    outs = []
    for pre in (False, True):
        layer = moe.FusedMoE(T, d["H"], d["I"], d["E"], d["topk"], d["w13"], d["w2"], d["w13_scale"],
                             d["w2_scale"], a_dtype=d["x"].dtype, out_dtype=w.out_dtype, device=DEV,
                             prequant=pre)
        assert layer.prequant == pre
        outs.append((layer(d["x"], d["logits"]).clone(), layer.act_scales().clone()))
        torch.cuda.synchronize()
    H.say(f"  {wl} T={T}: scales {outs[0][1].tolist()} / {outs[1][1].tolist()}")
    assert torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][0], outs[1][0])


def test_prequantised_step_in_a_graph():
    """The step with pre-quantised activations (routing, codes, forward)
    captured once and replayed with eager work in between: every replay
    equals the eager step."""
    w = W["decode_fp8"]
    T = 16
    d = inputs.make_inputs(w, T, device=DEV, seed=44)
    layer = moe.FusedMoE(T, w.H, w.I, w.E, w.topk, d["w13"], d["w2"], d["w13_scale"], d["w2_scale"],
                         a_dtype=d["x"].dtype, out_dtype=w.out_dtype, device=DEV, prequant=True)
    assert layer.prequant
    eager = layer(d["x"], d["logits"]).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            layer(d["x"], d["logits"], stream=s)
    torch.cuda.synchronize()
    for r in range(3):
        layer.out.zero_()
        layer.xq.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, eager), r
    del g


class _Events:
    """Raw hipEvent_t handles, created and read through the HIP runtime."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.h = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.h.append(e.value)

    def record(self, i, stream):
        assert self.hip.hipEventRecord(self.ct.c_void_p(self.h[i]),
                                       self.ct.c_void_p(stream.cuda_stream)) == 0

    def ms(self, a, b):
        v = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(v), self.ct.c_void_p(self.h[a]),
                                          self.ct.c_void_p(self.h[b]))
        assert rc == 0, rc
        return v.value

    def close(self):
        for e in self.h:
            self.hip.hipEventDestroy(self.ct.c_void_p(e))


@pytest.mark.parametrize("wl,T", [("decode_fp8", 16), ("prefill_bf16", 1100)])
def test_profiled_step_in_a_graph_records_its_events(wl, T):
    """The step with the library's kernel events (moe_fused_forward_profiled)
    captured in a graph: the events become event-record nodes that every
    replay re-records, so the GEMM durations read after each replay are
    positive and together fit inside the replay's own bracket, and the
    output equals the eager step's."""
    w = W[wl]
    kw = {} if wl == "decode_fp8" else dict(H=512, I=256, E=16, topk=4)
    d = inputs.make_inputs(w, T, device=DEV, seed=45, **kw)
    H_, I_, E_, k_ = d["H"], d["I"], d["E"], d["topk"]
    layer = moe.FusedMoE(T, H_, I_, E_, k_, d["w13"], d["w2"], d["w13_scale"], d["w2_scale"],
                         a_dtype=d["x"].dtype, out_dtype=w.out_dtype, device=DEV)
    ev = _Events(6)
    eager = layer(d["x"], d["logits"], events=ev.h[:4]).clone()
    torch.cuda.synchronize()
    assert ev.ms(0, 1) > 0 and ev.ms(2, 3) > 0  # eager records
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            layer(d["x"], d["logits"], stream=s, events=ev.h[:4])
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    for r in range(3):
        layer.out.zero_()
        torch.cuda.synchronize()
        ev.record(4, st)
        g.replay()
        ev.record(5, st)
        torch.cuda.synchronize()
        assert torch.equal(layer.out, eager), r
        g1, g2, whole = ev.ms(0, 1), ev.ms(2, 3), ev.ms(4, 5)
        assert g1 > 0 and g2 > 0 and g1 + g2 <= whole, (r, g1, g2, whole)
        assert ev.ms(4, 0) >= 0 and ev.ms(3, 5) >= 0, r  # inside this replay's bracket
    del g
    ev.close()


def _e4m3_positive_values():
    """The 127 non-negative finite E4M3FN values, ascending."""
    return np.array(sorted({float(oracle.e4m3_to_f64(c)) for c in range(0x7F)}), np.float64)


@pytest.mark.parametrize("s", [1.0, 0.37, 3.0e-3])
def test_quantize_codes_at_every_e4m3_midpoint(s):
    """Every rounding midpoint between adjacent E4M3 values (2^-10 between
    0 and the smallest subnormal among them), times the scale, and its fp32
    neighbours, both signs, plus values past saturation: the codes of the
    corrected-reciprocal quotient and the hardware conversion equal the
    oracle's E4M3(fl32(x / s)) with an IEEE division, bit for bit.  With
    s = 1 every quotient is exact (the conversion alone is pinned)."""
    v = _e4m3_positive_values()
    mids = (v[:-1] + v[1:]) / 2
    base = np.concatenate([mids, v, [448.0, 460.0, 464.0, 480.0, 1e4]])
    xs = []
    for m in base:
        f = np.float32(m * s)
        xs += [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf)),
               np.nextafter(np.nextafter(f, np.float32(np.inf)), np.float32(np.inf))]
    x = np.array(xs, np.float32)
    x = np.concatenate([x, -x, np.float32([0.0, -0.0])])
    x = np.concatenate([x, np.zeros((-len(x)) % 128, np.float32)])
    xd = torch.from_numpy(x).to(DEV)
    st = torch.tensor([s], dtype=torch.float32, device=DEV)
    codes, sc = moe.moe_quantize_act(xd, static_scale=st)
    torch.cuda.synchronize()
    ref = oracle.quantize_e4m3(x, float(np.float32(s)))
    got = codes.cpu().numpy()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(ref[i])) for i in bad[:8]]
