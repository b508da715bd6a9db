"""ctypes binding of the test-only probe library (libmoe_probe.so): the expert
GEMM kernels run on caller-built operands, gate/up sums stored raw."""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_probe.so")
DT = {torch.float32: 0, torch.bfloat16: 1, torch.float8_e4m3fn: 2}
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        import mixture_experts_layer_13_amd.moe  # noqa: F401  (HIP runtime of torch first)
        _lib = ctypes.CDLL(LIB_PATH)
        i, p = ctypes.c_int, ctypes.c_void_p
        _lib.moe_probe_gate_up.argtypes = [i] * 8 + [p] * 10 + [i, p]
        _lib.moe_probe_down.argtypes = [i] * 9 + [p] * 12 + [i, p]
    return _lib


def _p(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def gate_up(M, K, N, E, topk, block_m, max_blocks, x, w13, w13_scale, sx, al, hmax, gu, family):
    rc = lib().moe_probe_gate_up(M, K, N, E, topk, block_m, max_blocks, DT[w13.dtype], _p(x), _p(w13),
                                 _p(w13_scale), _p(sx), _p(al.sorted_pair_ids), _p(al.block_expert_ids),
                                 _p(al.expert_offsets), _p(al.num_padded), _p(hmax), _p(gu), family,
                                 _stream())
    assert rc == 0, rc


def down(M, K, N, E, topk, block_m, max_blocks, h, w2, w2_scale, sh, topk_w, al, y, out, family):
    rc = lib().moe_probe_down(M, K, N, E, topk, block_m, max_blocks, DT[w2.dtype], DT[out.dtype], _p(h),
                              _p(w2), _p(w2_scale), _p(sh), _p(topk_w), _p(al.sorted_pair_ids),
                              _p(al.block_expert_ids), _p(al.expert_offsets), _p(al.pair_pos),
                              _p(al.num_padded), _p(y), _p(out), family, _stream())
    assert rc == 0, rc
