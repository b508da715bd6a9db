"""Thin ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, and a non-zero status raises MoEError.  Every
step of the layer runs in the library's HIP kernels; there is no fallback.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN = 0, 1, 2, 3, 4
MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = 5, 6, 7
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2

EXPORTS = ("moe_status_string", "moe_last_error", "moe_align_capacity", "moe_workspace_size",
           "moe_route_topk", "moe_align_permute", "moe_fused_forward", "moe_quantize_act",
           "moe_fused_forward_profiled", "moe_fused_forward_noalloc", "moe_route_align", "moe_route_project_topk",
           "moe_route_project_workspace_size", "moe_rope_quantize_per_head", "moe_rope_workspace_size",
           "moe_fused_forward_persistent")
MOE_QUANT_WORKSPACE_BYTES = 8192
MOE_WORKSPACE_SCALES_OFFSET = 4096
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_FUSED_SYNC_BYTES = 32768
MOE_FUSED_SYNC_ERROR_OFFSET = 128


class MoEError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{moe_status_string(status)}: {detail}")


class moe_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("M", "K", "N", "E", "topk", "block_m", "a_dtype", "w_dtype", "out_dtype")]


_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_align_capacity.argtypes = [i32, i32, i32, i32]
        L.moe_align_capacity.restype = i64
        L.moe_workspace_size.argtypes = [ctypes.POINTER(moe_problem), ctypes.POINTER(sz)]
        L.moe_workspace_size.restype = ctypes.c_int
        L.moe_route_topk.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
        L.moe_route_topk.restype = ctypes.c_int
        L.moe_align_permute.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_align_permute.restype = ctypes.c_int
        L.moe_fused_forward.argtypes = [ctypes.POINTER(moe_problem)] + [vp] * 15 + [sz, vp]
        L.moe_fused_forward.restype = ctypes.c_int
        L.moe_quantize_act.argtypes = [vp, i32, i64, vp, vp, vp, vp, sz, vp]
        L.moe_quantize_act.restype = ctypes.c_int
        L.moe_fused_forward_profiled.argtypes = ([ctypes.POINTER(moe_problem)] + [vp] * 15 +
                                                 [sz, vp, ctypes.POINTER(ctypes.c_void_p)])
        L.moe_fused_forward_profiled.restype = ctypes.c_int
        L.moe_fused_forward_noalloc.argtypes = [ctypes.POINTER(moe_problem)] + [vp] * 15
        L.moe_fused_forward_noalloc.restype = ctypes.c_int
        L.moe_fused_forward_persistent.argtypes = ([ctypes.POINTER(moe_problem)] + [vp] * 15 +
                                                   [sz, vp, sz, vp])
        L.moe_fused_forward_persistent.restype = ctypes.c_int
        L.moe_route_align.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
        L.moe_route_align.restype = ctypes.c_int
        L.moe_route_project_topk.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, vp, vp,
                                             vp, vp, sz, vp]
        L.moe_route_project_topk.restype = ctypes.c_int
        L.moe_route_project_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        L.moe_route_project_workspace_size.restype = ctypes.c_int
        L.moe_rope_quantize_per_head.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp,
                                                 vp, vp, sz, vp]
        L.moe_rope_quantize_per_head.restype = ctypes.c_int
        L.moe_rope_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        L.moe_rope_workspace_size.restype = ctypes.c_int
        _lib = L
    return _lib


def moe_status_string(status):
    return lib().moe_status_string(int(status)).decode()


def moe_last_error():
    return lib().moe_last_error().decode()


def _check(status):
    if status != MOE_OK:
        raise MoEError(status, moe_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def dtype_code(dt):
    return {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16,
            torch.float8_e4m3fn: MOE_FP8_E4M3}[dt]


def moe_align_capacity(M, topk, E, block_m):
    return int(lib().moe_align_capacity(M, topk, E, block_m))


def make_problem(M, K, N, E, topk, block_m, a_dtype, w_dtype, out_dtype):
    return moe_problem(M, K, N, E, topk, block_m, dtype_code(a_dtype), dtype_code(w_dtype),
                       dtype_code(out_dtype))


def moe_workspace_size(problem):
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(problem), ctypes.byref(n)))
    return int(n.value)


def moe_route_project_workspace_size(M, K, E):
    n = ctypes.c_size_t(0)
    _check(lib().moe_route_project_workspace_size(M, K, E, ctypes.byref(n)))
    return n.value


def moe_route_project_topk(x, w_router, topk, renormalize=True, logits=None, topk_ids=None,
                           topk_weights=None, workspace=None, stream=None):
    """x [M,K] and w_router [E,K] (device, both bf16 or both f32) -> (ids
    int32 [M,k], weights f32 [M,k]); logits f32 [M,E] is written if given."""
    M, K = x.shape
    E = w_router.shape[0]
    if topk_ids is None:
        topk_ids = torch.empty(M, topk, dtype=torch.int32, device=x.device)
    if topk_weights is None:
        topk_weights = torch.empty(M, topk, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(moe_route_project_workspace_size(M, K, E), 16),
                                dtype=torch.uint8, device=x.device)
    _check(lib().moe_route_project_topk(_ptr(x), dtype_code(x.dtype), _ptr(w_router),
                                        dtype_code(w_router.dtype), M, K, E, topk,
                                        int(bool(renormalize)), _ptr(logits), _ptr(topk_ids),
                                        _ptr(topk_weights), _ptr(workspace), workspace.numel(),
                                        _stream(stream)))
    return topk_ids, topk_weights


def moe_route_topk(logits, topk, renormalize=True, topk_ids=None, topk_weights=None,
                   stream=None):
    """logits f32 [M,E] (device) -> (ids int32 [M,k], weights f32 [M,k])."""
    M, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty(M, topk, dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty(M, topk, dtype=torch.float32, device=logits.device)
    _check(lib().moe_route_topk(_ptr(logits), M, E, topk, int(bool(renormalize)),
                                _ptr(topk_ids), _ptr(topk_weights), _stream(stream)))
    return topk_ids, topk_weights


def moe_quantize_act(x, static_scale=None, codes=None, scale=None, workspace=None,
                     stream=None):
    """x f32/bf16 (device) -> (E4M3 codes as uint8, f32 scale [1])."""
    n = x.numel()
    dev = x.device
    codes = torch.empty(x.shape, dtype=torch.uint8, device=dev) if codes is None else codes
    scale = torch.empty(1, dtype=torch.float32, device=dev) if scale is None else scale
    if workspace is None:
        workspace = torch.empty(MOE_QUANT_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    _check(lib().moe_quantize_act(_ptr(x), dtype_code(x.dtype), n, _ptr(static_scale),
                                  _ptr(codes), _ptr(scale), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _stream(stream)))
    return codes, scale


def moe_fused_forward_noalloc(problem, x, w13, w2, topk_weights, alignment, out,
                              w13_scale=None, w2_scale=None, a1_scale=None, a2_scale=None,
                              stream=None):
    """moe_fused_forward on the library's own per-device scratch array (no
    workspace argument; nothing is allocated by the call)."""
    _check(lib().moe_fused_forward_noalloc(
        ctypes.byref(problem), _ptr(x), _ptr(w13), _ptr(w2), _ptr(w13_scale), _ptr(w2_scale),
        _ptr(a1_scale), _ptr(a2_scale), _ptr(topk_weights), _ptr(alignment.sorted_pair_ids),
        _ptr(alignment.block_expert_ids), _ptr(alignment.expert_offsets),
        _ptr(alignment.pair_pos), _ptr(alignment.num_padded), _ptr(out), _stream(stream)))
    return out


def moe_rope_workspace_size(T, n_heads, head_dim):
    n = ctypes.c_size_t(0)
    _check(lib().moe_rope_workspace_size(T, n_heads, head_dim, ctypes.byref(n)))
    return int(n.value)


def moe_rope_quantize_per_head(x, positions, inv_freq, interleaved=False, inverse=False,
                               static_scales=None, codes=None, scales=None, workspace=None,
                               stream=None):
    """x [T, nH, D] bf16/f32, positions int32 [T], inv_freq f32 [D/2] (device)
    -> (E4M3 codes uint8 [T, nH, D], scales f32 [nH])."""
    T, nH, D = x.shape
    dev = x.device
    codes = torch.empty(x.shape, dtype=torch.uint8, device=dev) if codes is None else codes
    scales = torch.empty(nH, dtype=torch.float32, device=dev) if scales is None else scales
    if workspace is None:
        workspace = torch.empty(max(moe_rope_workspace_size(T, nH, D), 16), dtype=torch.uint8,
                                device=dev)
    _check(lib().moe_rope_quantize_per_head(
        _ptr(x), dtype_code(x.dtype), _ptr(positions), _ptr(inv_freq), T, nH, D,
        int(bool(interleaved)), int(bool(inverse)), _ptr(static_scales), _ptr(codes),
        _ptr(scales), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return codes, scales


@dataclass
class Alignment:
    sorted_pair_ids: torch.Tensor
    block_expert_ids: torch.Tensor
    expert_offsets: torch.Tensor
    pair_pos: torch.Tensor
    num_padded: torch.Tensor
    block_m: int


def alloc_alignment(M, topk, E, block_m, device):
    cap = max(moe_align_capacity(M, topk, E, block_m), 1)
    i32 = dict(dtype=torch.int32, device=device)
    return Alignment(torch.empty(cap, **i32), torch.empty((cap + block_m - 1) // block_m, **i32),
                     torch.empty(E + 1, **i32), torch.empty(max(M * topk, 1), **i32),
                     torch.empty(1, **i32), block_m)


def moe_align_permute(topk_ids, E, block_m, workspace, alignment=None, stream=None):
    M, topk = topk_ids.shape
    al = alignment or alloc_alignment(M, topk, E, block_m, topk_ids.device)
    _check(lib().moe_align_permute(_ptr(topk_ids), M, topk, E, block_m,
                                   _ptr(al.sorted_pair_ids), _ptr(al.block_expert_ids),
                                   _ptr(al.expert_offsets), _ptr(al.pair_pos),
                                   _ptr(al.num_padded), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _stream(stream)))
    return al


def moe_route_align(logits, topk, renormalize, block_m, workspace, topk_ids=None,
                    topk_weights=None, alignment=None, stream=None):
    """Routing and alignment (one launch for M*topk <= 1024)."""
    M, E = logits.shape
    dev = logits.device
    if topk_ids is None:
        topk_ids = torch.empty(M, topk, dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty(M, topk, dtype=torch.float32, device=dev)
    al = alignment or alloc_alignment(M, topk, E, block_m, dev)
    _check(lib().moe_route_align(_ptr(logits), M, E, topk, int(bool(renormalize)), block_m,
                                 _ptr(topk_ids), _ptr(topk_weights), _ptr(al.sorted_pair_ids),
                                 _ptr(al.block_expert_ids), _ptr(al.expert_offsets),
                                 _ptr(al.pair_pos), _ptr(al.num_padded), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))
    return topk_ids, topk_weights, al


def moe_fused_forward(problem, x, w13, w2, topk_weights, alignment, out, workspace,
                      w13_scale=None, w2_scale=None, a1_scale=None, a2_scale=None,
                      stream=None, events=None):
    """events: None, or four hipEvent_t handles (ints or None) recorded around
    the two GEMM launches (moe_fused_forward_profiled)."""
    args = (ctypes.byref(problem), _ptr(x), _ptr(w13), _ptr(w2), _ptr(w13_scale),
            _ptr(w2_scale), _ptr(a1_scale), _ptr(a2_scale), _ptr(topk_weights),
            _ptr(alignment.sorted_pair_ids), _ptr(alignment.block_expert_ids),
            _ptr(alignment.expert_offsets), _ptr(alignment.pair_pos),
            _ptr(alignment.num_padded), _ptr(out), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if events is None:
        _check(lib().moe_fused_forward(*args))
    else:
        ev = (ctypes.c_void_p * 4)(*[(e or None) for e in events])
        _check(lib().moe_fused_forward_profiled(*args, ev))
    return out


def alloc_fused_sync(device="cuda"):
    """A zeroed synchronisation buffer for moe_fused_forward_persistent (one
    per stream; every call leaves it ready for the next)."""
    return torch.zeros(MOE_FUSED_SYNC_BYTES, dtype=torch.uint8, device=device)


def fused_sync_error(sync):
    """The error word of a synchronisation buffer (nonzero: a grid-wide wait
    of an earlier call gave up); reads the device, so it synchronises."""
    o = MOE_FUSED_SYNC_ERROR_OFFSET
    return int(sync[o:o + 4].view(torch.int32).item())


def moe_fused_forward_persistent(problem, x, w13, w2, topk_weights, alignment, out, workspace,
                                 sync, w13_scale=None, w2_scale=None, a1_scale=None,
                                 a2_scale=None, stream=None):
    """moe_fused_forward for E4M3 decode batches in one kernel launch; sync is
    a zero-initialised MOE_FUSED_SYNC_BYTES buffer (alloc_fused_sync)."""
    _check(lib().moe_fused_forward_persistent(
        ctypes.byref(problem), _ptr(x), _ptr(w13), _ptr(w2), _ptr(w13_scale), _ptr(w2_scale),
        _ptr(a1_scale), _ptr(a2_scale), _ptr(topk_weights), _ptr(alignment.sorted_pair_ids),
        _ptr(alignment.block_expert_ids), _ptr(alignment.expert_offsets),
        _ptr(alignment.pair_pos), _ptr(alignment.num_padded), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(sync),
        sync.numel() * sync.element_size(), _stream(stream)))
    return out


class FusedMoE:
    """The three calls with their buffers allocated once for a fixed maximum
    M (route -> align -> forward).  Buffers are reused between calls, so
    nothing is allocated or synchronised per call and the sequence can be
    captured into a HIP graph."""

    def __init__(self, M, K, N, E, topk, w13, w2, w13_scale=None, w2_scale=None,
                 block_m=None, a_dtype=torch.bfloat16, out_dtype=torch.bfloat16,
                 renormalize=True, a1_scale=None, a2_scale=None, device="cuda",
                 persistent=False, prequant=None):
        if block_m is None:
            # alignment block: 16 rows for decode-sized batches (the stream and
            # ring kernels), 256 once the experts average 512 rows or more (the
            # 256 x 256 prefill tiles), else 128
            block_m = 16 if M <= 64 else (256 if M * topk >= 512 * E else 128)
        self.M, self.K, self.N, self.E, self.topk = M, K, N, E, topk
        self.block_m, self.renormalize = block_m, renormalize
        self.w13, self.w2, self.w13_scale, self.w2_scale = w13, w2, w13_scale, w2_scale
        self.a1_scale, self.a2_scale = a1_scale, a2_scale
        self.problem = make_problem(M, K, N, E, topk, block_m, a_dtype, w13.dtype, out_dtype)
        ws = moe_workspace_size(self.problem)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=device)
        self.topk_ids = torch.empty(M, topk, dtype=torch.int32, device=device)
        self.topk_weights = torch.empty(M, topk, dtype=torch.float32, device=device)
        self.alignment = alloc_alignment(M, topk, E, block_m, device)
        self.out = torch.empty(M, K, dtype=out_dtype, device=device)
        # persistent: the forward runs as one launch (moe_fused_forward_persistent);
        # prequant (E4M3 weights; default: with the one launch only): the
        # activation codes are made by moe_quantize_act right after the
        # routing, and the forward starts from them (the one launch then
        # starts at gate/up)
        self.persistent = persistent
        self.sync = alloc_fused_sync(device) if persistent else None
        if prequant is None:
            prequant = persistent
        self.prequant = bool(prequant) and w13.dtype == torch.float8_e4m3fn
        if self.prequant:
            self.problem_q = make_problem(M, K, N, E, topk, block_m, torch.float8_e4m3fn,
                                          w13.dtype, out_dtype)
            self.xq = torch.empty(M, K, dtype=torch.uint8, device=device)
            self.xscale = torch.empty(1, dtype=torch.float32, device=device)
            self.qws = torch.empty(MOE_QUANT_WORKSPACE_BYTES, dtype=torch.uint8, device=device)

    def act_scales(self):
        """Device view of the (s_x, s_h) fp32 pair that the last E4M3 forward
        left in the workspace (include/moe.h, MOE_WORKSPACE_SCALES_OFFSET)."""
        o = MOE_WORKSPACE_SCALES_OFFSET
        return self.workspace[o:o + 8].view(torch.float32)

    def __call__(self, x, logits, stream=None, events=None):
        self.prepare(x, logits, stream)
        return self.forward(x, stream, events)

    def prepare(self, x, logits, stream=None):
        """Routing and alignment; in prequant mode then the activation codes."""
        self.route(logits, stream)
        if self.prequant:
            self.quantize(x, stream)

    def route(self, logits, stream=None):
        moe_route_align(logits, self.topk, self.renormalize, self.block_m, self.workspace,
                        self.topk_ids, self.topk_weights, self.alignment, stream)

    def quantize(self, x, stream=None):
        """The activation codes and scale of x (prequant mode)."""
        moe_quantize_act(x, self.a1_scale, self.xq, self.xscale, self.qws, stream)

    def forward(self, x, stream=None, events=None):
        if self.prequant and self.persistent:
            moe_fused_forward_persistent(self.problem_q, self.xq, self.w13, self.w2,
                                         self.topk_weights, self.alignment, self.out,
                                         self.workspace, self.sync, self.w13_scale,
                                         self.w2_scale, self.xscale, self.a2_scale, stream)
        elif self.prequant:
            moe_fused_forward(self.problem_q, self.xq, self.w13, self.w2, self.topk_weights,
                              self.alignment, self.out, self.workspace, self.w13_scale,
                              self.w2_scale, self.xscale, self.a2_scale, stream, events)
        elif self.persistent:
            moe_fused_forward_persistent(self.problem, x, self.w13, self.w2, self.topk_weights,
                                         self.alignment, self.out, self.workspace, self.sync,
                                         self.w13_scale, self.w2_scale, self.a1_scale,
                                         self.a2_scale, stream)
        else:
            moe_fused_forward(self.problem, x, self.w13, self.w2, self.topk_weights,
                              self.alignment, self.out, self.workspace, self.w13_scale,
                              self.w2_scale, self.a1_scale, self.a2_scale, stream, events)
        return self.out
