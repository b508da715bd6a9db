"""The launch path across batch sizes: no compilation, allocation or host
synchronisation for any M (the pages' JIT lesson, "Triton JIT recompilation
elimination": a new num_tokens must not trigger work on the host).

One set of buffers, sized for the largest M of the sweep, serves every M
(views of it).  A cold pass times the first call at each new M next to the
steady calls (no compile step: the first call costs about what later calls
cost, a kernel family's code-object loading included).  A warm pass checks,
per M, that the route -> align -> forward calls do not lower the device's
free memory (the library allocates nothing) and that they capture into
a HIP graph (capture fails on any synchronisation) whose replays equal the
eager result bit for bit; the eager result of every M is checked against
the fp64 oracle (every token up to M = 16, else the token of the last real
pair of every expert segment plus a seeded fill; E4M3 with the dynamic h
scale against the oracle's all-pairs scale).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_13_amd import inputs, moe
from tests import harness as H

pytestmark = pytest.mark.gpu

DEV = "cuda"
SWEEP = [1, 2, 3, 7, 8, 9, 16, 33, 63, 64, 65, 127, 200, 513, 1024, 2047, 4096, 8192]


def _block_m(M, k, E):
    return 16 if M <= 64 else (256 if M * k >= 512 * E else 128)


@pytest.mark.parametrize("wl", ["decode_bf16", "decode_fp8"])
def test_launch_path_sweep(wl):
    w = inputs.WORKLOADS[wl]
    Hd, Id, E, k = 1024, 512, 64, 8
    Mmax = max(SWEEP)
    d = inputs.make_inputs(w, Mmax, device=DEV, H=Hd, I=Id, E=E, topk=k)
    x, logits = d["x"], d["logits"]
    probs = {M: moe.make_problem(M, Hd, Id, E, k, _block_m(M, k, E), w.x_dtype, d["w13"].dtype,
                                 w.out_dtype) for M in SWEEP}
    ws_bytes = max(moe.moe_workspace_size(p) for p in probs.values())
    cap = max(moe.moe_align_capacity(M, k, E, _block_m(M, k, E)) for M in SWEEP)
    i32 = dict(dtype=torch.int32, device=DEV)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    ids_all = torch.empty(Mmax * k, **i32)
    wts_all = torch.empty(Mmax * k, dtype=torch.float32, device=DEV)
    sorted_all = torch.empty(cap, **i32)
    bexp_all = torch.empty(cap // 16 + 1, **i32)
    offs = torch.empty(E + 1, **i32)
    ppos_all = torch.empty(Mmax * k, **i32)
    npad = torch.empty(1, **i32)
    out_all = torch.empty(Mmax * Hd, dtype=w.out_dtype, device=DEV)

    def views(M):
        bm = _block_m(M, k, E)
        c = moe.moe_align_capacity(M, k, E, bm)
        al = moe.Alignment(sorted_all[:c], bexp_all[:(c + bm - 1) // bm], offs,
                           ppos_all[:M * k], npad, bm)
        return (bm, al, ids_all[:M * k].view(M, k), wts_all[:M * k].view(M, k),
                out_all[:M * Hd].view(M, Hd))

    def step(M, stream=None):
        bm, al, ids, wts, out = views(M)
        moe.moe_route_align(logits[:M], k, True, bm, ws, topk_ids=ids, topk_weights=wts,
                            alignment=al, stream=stream)
        moe.moe_fused_forward(probs[M], x[:M], d["w13"], d["w2"], wts, al, out, ws,
                              w13_scale=d["w13_scale"], w2_scale=d["w2_scale"], stream=stream)
        return out

    torch.cuda.synchronize()
    # pass 1, cold: the first call at each new M (in sweep order, so a new
    # kernel family's code-object loading lands in its first M), then steady
    rows = []
    for M in SWEEP:
        t0 = time.perf_counter()
        step(M)
        torch.cuda.synchronize()
        first = time.perf_counter() - t0
        steady = []
        for _ in range(5):
            t0 = time.perf_counter()
            step(M)
            torch.cuda.synchronize()
            steady.append(time.perf_counter() - t0)
        st = float(np.median(steady))
        rows.append((M, first * 1e3, st * 1e3))
    H.say("  M      first call ms   steady ms")
    for M, f, s_ in rows:
        H.say(f"  {M:5d}  {f:10.3f}  {s_:10.3f}")
    # a run-time compile costs hundreds of ms; the first call stays within a
    # few steady calls plus the upload of a kernel family's code object (4 ms
    # for the process's first launches on MI355X; 50 ms of margin for a cold
    # box)
    for M, f, s_ in rows:
        assert f < 3 * s_ + 50.0, (M, f, s_)
    # pass 2, warm: no device memory is allocated by the calls, and they
    # capture into a graph (no synchronisation) whose replays are bit-exact
    for M in SWEEP:
        free0 = torch.cuda.mem_get_info()[0]
        step(M)
        torch.cuda.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
        # an allocation would lower the free memory; it may rise when the
        # runtime releases an earlier size's graph in the meantime
        assert free1 >= free0, (M, free0, free1)
        eager = views(M)[4].clone()
        # the eager result against the oracle
        dm = dict(d, x=x[:M], logits=logits[:M], T=M)
        rids, _ = oracle.route_topk(logits[:M].cpu().numpy(), k, True)
        assert np.array_equal(views(M)[2].cpu().numpy(), rids), M
        tokens = H.sample_tokens(rids, 16, seed=M)
        if w.fp8_act:
            o = moe.MOE_WORKSPACE_SCALES_OFFSET
            H.check_fp8_dynamic(dm, ws[o:o + 8].view(torch.float32), eager, tokens, f"M={M}")
        else:
            ref, _, _, _ = H.oracle_forward(dm, tokens=tokens)
            err = H.row_rel_err(H.to_f64(eager)[tokens], ref)
            H.say(f"  M={M}: {len(tokens)} rows, max row rel err {err:.3e}")
            assert err <= H.BF16_TOL, (M, err)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                step(M, stream=s)
        torch.cuda.synchronize()
        for _ in range(2):
            views(M)[4].zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(views(M)[4], eager), M
        del g
