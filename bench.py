"""Fused-MoE layer benchmark on one MI355X.

A step is one pass of the whole layer -- route -> align -> gate/up GEMM ->
SiLU * up -> down GEMM -> weighted combine -- over one batch of seeded
synthetic input already resident in HBM.  Default workload: prefill bf16,
T=8192 tokens, H=4096, I=1024, E=64, top-8 with Zipf(1.1)-skewed routing,
the largest single-GPU configuration (the most tokens and flops);
--workload / --tokens select the others.

Prints one JSON line: tokens/s for the whole job (median of K replays of
the step captured in a HIP graph, each replay after a 512 MiB read that
evicts the L2s and the MALL; median, p10 and p90 in "timed", back-to-back
replays in "warm"), the roofline of the
dominant kernel (the gate/up GEMM, HIP events around its launch inside the
timed steps) and the fp64 CPU oracle timed on a bounded sample of the same
batch on the host's cores.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 2500.0, "e4m3": 5000.0}
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "pmc_mfma.json")
# Sources of the gate/up kernel each stored counter record was taken with,
# per kernel family (counters go stale when these change).
_CSRC = os.path.join(ROOT, "mixture_experts_layer_13_amd", "csrc")
KERNEL_SRCS = {
    "decode": ["ring.hip", "ring.hpp", "fused.hip", "gemm.hip", "common.hpp", "launch.hpp"],
    "prefill": ["prefill.hip", "prefill2.hip", "gemm.hip", "common.hpp", "launch.hpp"],
}


# The pages' own figures, quoted as context: relative gains measured on NVIDIA
# H200 inside a serving stack; the pages give no absolute throughput, so no
# figure here is comparable with this line's value.
PAGES_H200 = {
    "end_to_end_throughput_gain": "up to 10% (the three optimisations together; FP8 decode routed to the fused backend)",
    "swap_ab_gain": "2-4% end-to-end (decode)",
    "ttft_gain_no_jit_recompile": "9% (prefill, RoPE + per-head FP8 kernel; not this layer)",
    "hardware": "NVIDIA H200",
}


def kernel_source_sha(family):
    """SHA-256 over the sources of one GEMM kernel family."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS[family]:
        h.update(open(os.path.join(_CSRC, f), "rb").read())
    return h.hexdigest()


class CacheFlush:
    """Evicts the L2s and the 256 MB MALL before a timed step by reading a
    512 MiB buffer (a max-reduction into one word).  A read leaves the caches
    holding clean lines.  A write of the same size (write(), the control)
    leaves them dirty, and the step timed after it also pays for writing
    those lines back to HBM."""

    BYTES = 512 << 20

    def __init__(self, dev):
        import torch

        self.torch = torch
        self.buf = torch.full((self.BYTES // 4,), 3, dtype=torch.int32, device=dev)
        self.sink = torch.empty((), dtype=torch.int32, device=dev)

    def __call__(self):
        self.torch.amax(self.buf, dim=0, out=self.sink)

    def write(self, v):
        self.buf.fill_(v)


def dense_gemm_context(layer, wl, H, I, dev, reps=20):
    """The vendor library's dense GEMM (hipBLASLt through torch.mm, E4M3
    through torch._scaled_mm) on the shapes the expert GEMMs execute: all
    padded rows of this batch against one weight matrix of the gate/up
    [2I, H] and down [H, I] products, each timed after the same 512 MiB flush
    (median of `reps`).  A calibration of what a tuned dense GEMM reaches on
    this chip at its clock under load, not a result of the layer."""
    import torch

    rows = int(layer.alignment.num_padded.item())
    flush = CacheFlush(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    out = {"library": "hipBLASLt (torch.mm; E4M3: torch._scaled_mm)", "rows": rows}
    for name, (k_, n_) in (("gate_up", (H, 2 * I)), ("down", (I, H))):
        a = torch.randn(rows, k_, device=dev, dtype=torch.bfloat16, generator=g)
        b = torch.randn(n_, k_, device=dev, dtype=torch.bfloat16, generator=g)
        if wl.w_dtype == "e4m3":
            a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)
            one = torch.ones((), device=dev)

            def fn():
                return torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        else:
            def fn():
                return torch.mm(a, b.t())
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            flush()
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]
        out[name] = {"m_k_n": [rows, k_, n_], "tflops": round(2.0 * rows * k_ * n_ / (ms * 1e-3) / 1e12, 1)}
        del a, b
    del flush
    return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_bf16")
    ap.add_argument("--tokens", type=int, default=8192)
    ap.add_argument("--cpu-sample", type=int, default=64,
                    help="tokens of the batch the CPU oracle is timed on (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="host seconds the oracle timing aims at (repeats of the sample)")
    ap.add_argument("--router", action="store_true",
                    help="time the router projection fused with the routing "
                         "(moe_route_project_topk) on the workload's activations instead of the layer")
    ap.add_argument("--rope", action="store_true",
                    help="time the rotary embedding + per-head E4M3 kernel "
                         "(moe_rope_quantize_per_head) on x [tokens, 32 heads, 128] bf16 instead of the layer")
    ap.add_argument("--heads", type=int, default=32)
    ap.add_argument("--head-dim", type=int, default=128)
    ap.add_argument("--persistent", action="store_true",
                    help="E4M3 decode: run the forward as one launch (moe_fused_forward_persistent)")
    ap.add_argument("--in-kernel-x", action="store_true",
                    help="with --persistent: quantise x inside the one launch instead of beside the "
                         "routing")
    ap.add_argument("--copy-check", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own stream)."""

    def __init__(self):
        import ctypes
        import torch  # noqa: F401  (loads the HIP runtime torch uses)
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = self.ct.c_void_p()
            rc = self.hip.hipEventCreate(self.ct.byref(h))
            assert rc == 0, rc
            out.append(h.value)
        return out

    def record(self, e, stream):
        self.hip.hipEventRecord.argtypes = [self.ct.c_void_p, self.ct.c_void_p]
        rc = self.hip.hipEventRecord(self.ct.c_void_p(e), self.ct.c_void_p(stream))
        assert rc == 0, rc

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(a),
                                          self.ct.c_void_p(b))
        assert rc == 0, rc
        return ms.value


def read_clocks():
    """Current shader and memory clock levels from the driver's sysfs tables
    (the line the driver marks with '*'); plain file reads, no child
    process.  None where the tables are not readable."""
    import glob
    clk = {}
    for key, fname in (("sclk", "pp_dpm_sclk"), ("mclk", "pp_dpm_mclk"), ("fclk", "pp_dpm_fclk")):
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/{fname}")):
            try:
                for ln in open(path):
                    if ln.rstrip().endswith("*"):
                        clk.setdefault(key, ln.split(":", 1)[-1].strip(" *\n"))
            except OSError:
                pass
    return clk or None


def router_main(args):
    """Router projection (logits = x . W_r^T, W_r [E, H]) followed by the
    top-k routing (moe_route_project_topk: a K-split projection launch and a
    reduce-and-route launch), on the workload's activations and a seeded
    router weight of the same dtype.  Algorithmic bytes: x, W_r and the ids
    and weights (the partial sums between the two launches are not counted);
    the kernel time is that of the whole call."""
    import numpy as np
    import torch

    from mixture_experts_layer_13_amd import inputs, moe

    moe.lib()  # fail loudly if the HIP library is missing
    dev = "cuda"
    wl = inputs.WORKLOADS[args.workload]
    T = args.tokens
    d = inputs.make_inputs(wl, T, device=dev)
    H, E, k = d["H"], d["E"], d["topk"]
    x = d["x"]
    wr = inputs.make_router(E, H, 600 + E, x.dtype, device=dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    ws = torch.empty(max(moe.moe_route_project_workspace_size(T, H, E), 16), dtype=torch.uint8,
                     device=dev)
    K, W = args.steps, args.warmup
    for _ in range(W):
        moe.moe_route_project_topk(x, wr, k, True, topk_ids=ids, topk_weights=wts, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(K):
                moe.moe_route_project_topk(x, wr, k, True, topk_ids=ids, topk_weights=wts, workspace=ws)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    # kernel durations: events on the launch stream around each eager call,
    # queued behind one more replay
    ev = HipEvents()
    evs = ev.create(2 * K)
    st = torch.cuda.current_stream()
    graph.replay()
    for i in range(K):
        ev.record(evs[2 * i], st.cuda_stream)
        moe.moe_route_project_topk(x, wr, k, True, topk_ids=ids, topk_weights=wts, workspace=ws)
        ev.record(evs[2 * i + 1], st.cuda_stream)
    torch.cuda.synchronize()
    k_ms = sum(ev.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(K)) / K
    b = x.element_size()
    alg = T * H * b + E * H * b + T * k * 8
    achieved = alg / (k_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "route_project_partial_kernel + route_project_reduce_kernel", "avg_launch_us": round(k_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": int(alg),
            "flop_per_launch": int(2 * T * H * E)}
    cpu = None
    if args.cpu_sample > 0:
        import oracle

        S = min(args.cpu_sample, T)
        xb = inputs.to_numpy_bits(x[:S])
        wb = inputs.to_numpy_bits(wr)
        c0 = time.perf_counter()
        oracle.route_project(xb, wb, k, True)
        once = time.perf_counter() - c0
        reps = max(1, int(np.ceil(args.cpu_seconds / max(once, 1e-3))))
        c0 = time.perf_counter()
        for _ in range(reps):
            oracle.route_project(xb, wb, k, True)
        wall = time.perf_counter() - c0
        cpu = {"value": round(S * reps / wall, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"first {S} tokens of the same batch (fp64 projection and routing), "
                         f"{reps} passes, {wall:.1f} s wall"}
    line = {
        "metric": "router projection + top-k routing tokens/s",
        "value": round(T / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {torch.bfloat16: "bf16", torch.float32: "f32"}[x.dtype],
        "data": "synthetic (seeded; no public dataset or trained weights on the pages)",
        "config": {"workload": f"router of {args.workload} T={T} H={H} E={E} top-{k}",
                   "tokens": T, "hidden": H, "experts": E, "topk": k},
        "timing": "K calls captured in one HIP graph, replayed between synchronisations; "
                  "kernel duration from HIP events around eager calls queued behind a replay",
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def rope_main(args):
    """Rotary position embedding fused with per-head E4M3 quantisation on
    x [T, heads, head_dim] bf16 ~ N(0, 1), positions 0..T-1, inverse
    frequencies 10000^(-2i/D).  Each of the K timed steps follows a 512 MiB
    flush and is bracketed by HIP events on the launch stream.  Algorithmic
    bytes: x read once, the codes written once, positions, frequencies and
    scales (the second read of x by the quantising pass is not counted)."""
    import numpy as np
    import torch

    from mixture_experts_layer_13_amd import inputs, moe

    moe.lib()  # fail loudly if the HIP library is missing
    dev = "cuda"
    T, nH, D = args.tokens, args.heads, args.head_dim
    x = inputs.make_x(T, nH * D, 4000 + T, torch.bfloat16, device=dev).view(T, nH, D)
    pos = torch.arange(T, dtype=torch.int32, device=dev)
    invf = torch.tensor((10000.0 ** (-np.arange(0, D, 2) / D)).astype(np.float32), device=dev)
    codes = torch.empty(T, nH, D, dtype=torch.uint8, device=dev)
    scales = torch.empty(nH, dtype=torch.float32, device=dev)
    ws = torch.empty(max(moe.moe_rope_workspace_size(T, nH, D), 16), dtype=torch.uint8, device=dev)

    def call():
        moe.moe_rope_quantize_per_head(x, pos, invf, codes=codes, scales=scales, workspace=ws)

    K, W = args.steps, args.warmup
    for _ in range(W):
        call()
    torch.cuda.synchronize()
    ev = HipEvents()
    st = torch.cuda.current_stream()
    flush = CacheFlush(dev)
    sev = ev.create(2 * K)
    torch.cuda.synchronize()
    for i in range(K):
        flush()
        ev.record(sev[2 * i], st.cuda_stream)
        call()
        ev.record(sev[2 * i + 1], st.cuda_stream)
    torch.cuda.synchronize()
    us = np.array([ev.elapsed_ms(sev[2 * i], sev[2 * i + 1]) for i in range(K)]) * 1e3
    med = float(np.median(us))
    # warm, for context: back-to-back calls in one graph
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(K):
                moe.moe_rope_quantize_per_head(x, pos, invf, codes=codes, scales=scales,
                                               workspace=ws, stream=cap)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    warm_us = (time.perf_counter() - w0) * 1e6 / K
    del graph, flush
    n = T * nH * D
    alg = n * (2 + 1) + T * 4 + (D // 2) * 4 + nH * 4
    achieved = alg / (med * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "rope_amax_kernel + rope_quant_kernel" if n > (1 << 15) else "rope_one_kernel",
            "avg_launch_us": round(float(us.mean()), 2), "algorithmic_bytes_per_launch": int(alg)}
    cpu = None
    if args.cpu_sample > 0:
        import oracle

        S = min(args.cpu_sample, T)
        xb = inputs.to_numpy_bits(x[:S])
        pb = pos[:S].cpu().numpy()
        fb = invf.cpu().numpy()
        c0 = time.perf_counter()
        oracle.rope_quant_per_head(xb, pb, fb)
        once = time.perf_counter() - c0
        reps = max(1, int(np.ceil(args.cpu_seconds / max(once, 1e-3))))
        c0 = time.perf_counter()
        for _ in range(reps):
            oracle.rope_quant_per_head(xb, pb, fb)
        wall = time.perf_counter() - c0
        cpu = {"value": round(S * reps / wall, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"first {S} tokens as a batch of their own (fp64 rotation, per-head "
                         f"scales, codes), {reps} passes, {wall:.1f} s wall"}
    line = {
        "metric": "rotary embedding + per-head E4M3 quantisation tokens/s",
        "value": round(T / (med * 1e-6), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(med * 1e-3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; no public dataset or trained weights on the pages)",
        "config": {"workload": f"rope_fp8 T={T} heads={nH} head_dim={D}", "tokens": T,
                   "heads": nH, "head_dim": D},
        "timing": "median of K calls, each after a 512 MiB write that evicts L2 and the MALL, "
                  "HIP events on the launch stream",
        "timed": {"median_us": round(med, 2), "p10_us": round(float(np.percentile(us, 10)), 2),
                  "p90_us": round(float(np.percentile(us, 90)), 2), "steps": K},
        "roofline": roof, "cpu_baseline": cpu,
        "warm": {"us_per_call": round(warm_us, 2)},
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer runs "
              "on one GPU: no collectives, no sharding)", file=sys.stderr)
        sys.exit(2)
    if args.router:
        router_main(args)
        return
    if args.rope:
        rope_main(args)
        return
    import numpy as np
    import torch

    from mixture_experts_layer_13_amd import inputs, moe

    moe.lib()  # fail loudly if the HIP library is missing
    dev = "cuda"
    wl = inputs.WORKLOADS[args.workload]
    T = args.tokens
    d = inputs.make_inputs(wl, T, device=dev)
    H, I, E, k = d["H"], d["I"], d["E"], d["topk"]
    layer = moe.FusedMoE(T, H, I, E, k, d["w13"], d["w2"], d["w13_scale"], d["w2_scale"],
                         a_dtype=wl.x_dtype, out_dtype=wl.out_dtype, device=dev,
                         persistent=args.persistent,
                         prequant=False if args.in_kernel_x else None)
    x, logits = d["x"], d["logits"]

    ev = HipEvents()
    K, W = args.steps, args.warmup
    st = torch.cuda.current_stream()
    flush = CacheFlush(dev)

    def profiled_step(kev):
        """route + align (+ the activation codes when x is quantised beside
        the routing) -> forward, with HIP events around the GEMM launches."""
        if args.persistent:  # the one launch of the forward between the kernel events
            layer.prepare(x, logits)
            ev.record(kev[0], st.cuda_stream)
            layer.forward(x)
            ev.record(kev[1], st.cuda_stream)
        else:
            layer(x, logits, events=kev)

    layer(x, logits)  # first call outside any capture (loads the kernels)
    torch.cuda.synchronize()
    # One step (route -> align -> forward) captured in a HIP graph.
    step_graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(st)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(step_graph, stream=cap):
            layer(x, logits)
    torch.cuda.synchronize()
    for _ in range(W):
        step_graph.replay()
        layer(x, logits)
    torch.cuda.synchronize()
    # Timed region: K rounds of four steps, each step after a 512 MiB read
    # that evicts the L2s and the 256 MB MALL (outside the step's events, so
    # every step reads its weights from HBM), each bracketed by HIP events on
    # the launch stream: a replay of the captured step (the headline), the
    # same calls enqueued eagerly, an eager step with the library's events
    # around its GEMM launches (the kernel durations; events between kernels
    # lengthen that step by a few us, so it is not the step time), and, as a
    # control, a replay after a 512 MiB write instead of the read (the step
    # then also writes the flush's dirty lines back).  The host queues the
    # next flush and steps while the GPU runs, so no step is host-paced.
    sev = ev.create(8 * K)
    kev = ev.create(4 * K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e8 = sev[8 * i: 8 * i + 8]
        flush()
        ev.record(e8[0], st.cuda_stream)
        step_graph.replay()
        ev.record(e8[1], st.cuda_stream)
        flush()
        ev.record(e8[2], st.cuda_stream)
        layer(x, logits)
        ev.record(e8[3], st.cuda_stream)
        flush()
        ev.record(e8[4], st.cuda_stream)
        profiled_step(kev[4 * i: 4 * i + 4])
        ev.record(e8[5], st.cuda_stream)
        flush.write(i & 0xFF)
        ev.record(e8[6], st.cuda_stream)
        step_graph.replay()
        ev.record(e8[7], st.cuda_stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    del step_graph

    def span_us(evs, stride, a, b):
        return np.array([ev.elapsed_ms(evs[stride * i + a], evs[stride * i + b])
                         for i in range(K)]) * 1e3

    def stats(us):
        return {"median_us": round(float(np.median(us)), 2),
                "p10_us": round(float(np.percentile(us, 10)), 2),
                "p90_us": round(float(np.percentile(us, 90)), 2)}

    step_us = span_us(sev, 8, 0, 1)
    g1_ms = float(span_us(kev, 4, 0, 1).mean()) * 1e-3
    g2_ms = 0.0 if args.persistent else float(span_us(kev, 4, 2, 3).mean()) * 1e-3
    med_us = float(np.median(step_us))
    ms_step = med_us * 1e-3
    timed = dict(stats(step_us), steps=K, warmup=W, flush_bytes=CacheFlush.BYTES,
                 protocol="replays of the step captured in one HIP graph, each after a 512 MiB read",
                 eager=stats(span_us(sev, 8, 2, 3)),
                 profiled_step=stats(span_us(sev, 8, 4, 5)),
                 replay_after_write_flush=stats(span_us(sev, 8, 6, 7)),
                 wall_s_all_four_incl_flushes=round(wall_s, 4))

    # Warm, for context: K steps captured once into a HIP graph and replayed
    # back to back (as a serving loop runs them); between steps the MALL keeps
    # the weights read last.
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(K):
                layer(x, logits)
    torch.cuda.synchronize()
    graph.replay()  # untimed: the first replay uploads the graph
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    warm_us = (time.perf_counter() - w0) * 1e6 / K
    del graph, flush
    warm = {"us_per_step": round(warm_us, 2), "tokens_per_s": round(T / (warm_us * 1e-6), 1),
            "timing": "K steps in one HIP graph, replayed back to back between synchronisations"}

    # context for the roofline: a plain device-to-device copy of 1 GiB (read
    # and write bytes counted) and the clocks the driver reports
    ca = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cb = torch.empty_like(ca)
    cb.copy_(ca)
    torch.cuda.synchronize()
    ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ce0.record()
    for _ in range(5):
        cb.copy_(ca)
    ce1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * (1 << 30) / (ce0.elapsed_time(ce1) * 1e-3) / 1e9
    del ca, cb
    context = {"d2d_copy_gbps": round(copy_gbps, 1), "clocks": read_clocks(),
               "pages_h200": PAGES_H200}
    if T > 64 and wl.w_dtype in ("bf16", "e4m3"):
        context["dense_gemm"] = dense_gemm_context(layer, wl, H, I, dev)

    if args.copy_check:  # plain copy of known size, for counter calibration
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    # algorithmic work of this batch (padding and re-reads excluded)
    ids = layer.topk_ids.cpu().numpy()
    U = int(len(np.unique(ids)))
    P = T * k
    bw = {"f32": 4, "bf16": 2, "e4m3": 1}[wl.w_dtype]
    bx = torch.tensor([], dtype=wl.x_dtype).element_size()
    bo = torch.tensor([], dtype=wl.out_dtype).element_size()
    fp8 = wl.w_dtype == "e4m3"
    bh = 4 if fp8 else 2
    op_bytes = U * 3 * H * I * bw + T * H * (bx + bo) + T * E * 4 + T * k * 8 + (8 * U if fp8 else 0)
    g1_bytes = U * 2 * I * H * bw + T * H * (1 if fp8 else bx) + P * I * bh + (4 * U if fp8 else 0)
    flops = 6.0 * T * k * H * I
    stream_path = T <= 64
    hbm_bound = (flops / op_bytes) < 300.0

    if args.persistent:
        # the dominant (only) kernel is the whole forward: its bytes are the
        # op's, less the routing's logits and ids, which the routing launch
        # reads (and, when x is quantised beside the routing, x itself: the
        # launch then reads its codes)
        g1_bytes = op_bytes - T * E * 4 - T * k * 8
        if layer.prequant:
            g1_bytes += T * H * (1 - bx)
    if hbm_bound:
        achieved = g1_bytes / (g1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        g1_flops = 4.0 * T * k * H * I
        achieved = g1_flops / (g1_ms * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[wl.w_dtype]
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None}
        # the flops the kernel executes, the padding rows of the alignment
        # blocks included (what the dense GEMM in "context" is comparable with)
        rows = int(layer.alignment.num_padded.item())
        roof["executed_tflops"] = round(4.0 * rows * H * I / (g1_ms * 1e-3) / 1e12, 2)
    ring = stream_path and wl.w_dtype in ("bf16", "e4m3") and (H * bw) % 512 == 0
    if args.persistent:
        roof["kernel"] = "fused_decode_kernel"
    elif stream_path:  # the gate/up instantiation of the persistent expert ring
        roof["kernel"] = "ring_gemm_kernel<W, NCB, 4, WPC, true>" if ring else "gemm1_stream_kernel"
    elif wl.w_dtype in ("bf16", "e4m3"):  # prefill kernels: 256 x 256 tiles with 256-row blocks
        roof["kernel"] = "pfq_gemm_kernel" if layer.block_m == 256 else "pf_gemm_kernel"
    else:
        roof["kernel"] = "gemm1_tile_kernel"
    roof["avg_launch_us"] = round(g1_ms * 1e3, 2)
    roof["algorithmic_bytes_per_launch"] = int(g1_bytes)
    src_sha = kernel_source_sha("decode" if (stream_path or args.persistent) else "prefill")
    key = f"{args.workload}:T{T}" + (":persistent" if args.persistent else "")
    if fp8:
        roof["x_quantised"] = ("beside the routing (moe_quantize_act)" if layer.prequant
                               else "inside the launch" if args.persistent else "by the forward")
    if os.path.exists(PMC_FILE):
        rec = json.load(open(PMC_FILE)).get(key)
        if rec and rec.get("gemm_source_sha256") == src_sha:
            roof["traffic"] = int(rec["hbm_bytes_per_launch"])
    if os.path.exists(MFMA_FILE):
        # MFMA work and busy cycles of the gate/up kernel from a separate
        # rocprofv3 --pmc pass over this same command (only while the GEMM
        # sources are the ones the counters were taken with)
        rec = json.load(open(MFMA_FILE)).get(key)
        if rec and rec.get("gemm_source_sha256") == src_sha:
            roof["mfma_counters"] = {k_: rec[k_] for k_ in (
                "kernel", "mops_per_dispatch", "flop_per_dispatch", "mfma_busy_frac",
                "clock_ghz", "counter_duration_us") if k_ in rec}

    cpu = None
    if args.cpu_sample > 0:
        import oracle

        # the oracle on the first S tokens of the same batch taken as a batch
        # of their own (routing, and for E4M3 the dynamic per-tensor scales of
        # x and h over these S tokens), repeated until about --cpu-seconds of
        # host work have been timed (one untimed pass first, which also sizes
        # the repeat count)
        S = min(args.cpu_sample, T)
        lg = logits.cpu().numpy()
        rids, rw = oracle.route_topk(lg, k, True)
        used = np.unique(rids[:S])
        remap = np.full(E, 0, np.int32)
        remap[used] = np.arange(len(used), dtype=np.int32)
        sel = torch.as_tensor(used, device=dev, dtype=torch.long)
        w13 = inputs.to_numpy_bits(d["w13"].index_select(0, sel))
        w2 = inputs.to_numpy_bits(d["w2"].index_select(0, sel))
        s13 = s2 = None
        if fp8:
            s13 = d["w13_scale"].index_select(0, sel).cpu().numpy()
            s2 = d["w2_scale"].index_select(0, sel).cpu().numpy()
        xb = inputs.to_numpy_bits(x)

        def oracle_pass():
            ro = oracle.route_topk(lg[:S], k, True)  # routing of the sample, timed
            return oracle.moe_forward(xb[:S], w13, w2, remap[ro[0]], ro[1], s13, s2,
                                      fp8_act=fp8)[0]

        c0 = time.perf_counter()
        ref = oracle_pass()
        once = time.perf_counter() - c0
        reps = max(1, int(np.ceil(args.cpu_seconds / max(once, 1e-3))))
        c0 = time.perf_counter()
        for _ in range(reps):
            oracle_pass()
        wall = time.perf_counter() - c0
        got = layer.out[:S].float().cpu().numpy().astype(np.float64)
        cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        cpu = {"value": round(S * reps / wall, 3), "unit": "tokens/s", "cores": cores,
               "kind": "oracle",
               "sample": f"first {S} tokens of the same batch as a batch of their own (routing + "
                         f"{S}x{k} expert pairs in fp64" + (", dynamic x and h scales over them" if fp8 else "")
                         + f"), {reps} passes, {wall:.1f} s wall"}
        if not fp8:  # (E4M3: the sub-batch has its own h scale, so rows are not comparable)
            err = float((np.abs(got - ref).max(1) / np.abs(ref).max(1)).max())
            cpu["sample_max_row_rel_err_vs_gpu"] = float(f"{err:.3e}")

    line = {
        "metric": "fused-MoE tokens/s + achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill)",
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "bf16", "e4m3": "fp8_e4m3"}[wl.w_dtype],
        "data": "synthetic (seeded; no public dataset or trained weights on the pages)",
        "config": {"workload": f"{args.workload} T={T} H={H} I={I} E={E} top-{k}",
                   "tokens": T, "hidden": H, "intermediate": I, "experts": E, "topk": k,
                   "active_experts": U, "block_m": layer.block_m,
                   "kernel_family": ("one launch" if args.persistent else
                                     "stream" if stream_path else "tile")},
        "op_hbm_gbps": round(op_bytes / (ms_step * 1e-3) / 1e9, 1),
        "op_tflops": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "down_gemm_avg_launch_us": None if args.persistent else round(g2_ms * 1e3, 2),
        "timing": "median of K replays of the step captured in one HIP graph, each after a "
                  "512 MiB read that evicts L2 and the MALL, timed with HIP events on the launch "
                  "stream; GEMM durations from the library's events around its launches in K "
                  "eager steps interleaved with the replays in the same timed region",
        "timed": timed,
        "roofline": roof,
        "cpu_baseline": cpu,
        "warm": warm,
        "gemm_source_sha256": src_sha[:16],
    }
    warm["op_hbm_gbps"] = round(op_bytes / (warm_us * 1e-6) / 1e9, 1)
    warm["op_tflops"] = round(flops / (warm_us * 1e-6) / 1e12, 3)
    line["context"] = context
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
