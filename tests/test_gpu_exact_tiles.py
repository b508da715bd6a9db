"""Integer-exact checks of the expert GEMM tiles (test-only probe library).

Operands are small integers (exact in bf16 and E4M3, scales 1), so every fp32
partial sum the MFMAs form is an exact integer below 2^24 and the kernels'
gate and up sums and down outputs must equal an integer matrix product bit for
bit, whatever the summation order.  This pins the operand placement of the
kernels -- weights on the MFMA row operand, tokens on the column operand, the
product read back as (A B)^T = B^T A^T ("Amazon SageMaker AI 上的
Mixture-of-Experts 内核工程优化", section "Swap-AB for WGMMA utilization") --
for every kernel family: decode ring and stream kernels (family 0) and the
tile kernels (family 1), bf16, E4M3 and f32 weights.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_13_amd import moe
from tests.probe import probe

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ints(shape, lo, hi, seed):
    g = np.random.default_rng(seed)
    return g.integers(lo, hi + 1, size=shape).astype(np.int64)


def _routing(M, E, k, seed):
    g = np.random.default_rng(seed)
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(M)]).astype(np.int32)
    return ids


def _setup(M, E, k, block_m, seed):
    ids = _routing(M, E, k, seed)
    ids_d = torch.as_tensor(ids, device=DEV)
    ws = torch.empty(1 << 24, dtype=torch.uint8, device=DEV)
    al = moe.moe_align_permute(ids_d, E, block_m, ws)
    cap = moe.moe_align_capacity(M, k, E, block_m)
    max_blocks = cap // min(block_m, 128)
    torch.cuda.synchronize()
    return ids, al, cap, max_blocks


def _to_dev(a, dtype):
    return torch.as_tensor(a.astype(np.float32), device=DEV).to(dtype)


# (family, weight dtype, M, K, N, E, k, block_m)
GATE_UP = [
    (0, torch.bfloat16, 5, 2048, 256, 8, 2, 16),     # ring, one column block
    (0, torch.bfloat16, 40, 2048, 256, 8, 2, 16),    # ring, two column blocks
    (0, torch.float8_e4m3fn, 40, 2048, 256, 8, 2, 16),
    (0, torch.bfloat16, 40, 2048, 256, 8, 2, 32),    # ring, 32-column token groups
    (0, torch.float8_e4m3fn, 64, 2048, 256, 8, 2, 64),  # two groups per 64-row block
    (0, torch.bfloat16, 1, 2048, 256, 8, 2, 16),     # fewer tasks than workgroups
    (0, torch.float32, 12, 512, 256, 8, 2, 16),      # stream kernel (f32 weights)
    (1, torch.bfloat16, 200, 1024, 256, 8, 2, 128),  # prefill kernel, 256 x 128 tiles
    (1, torch.float8_e4m3fn, 200, 1024, 256, 8, 2, 256),  # 256 x 256 tiles
    (1, torch.bfloat16, 300, 1024, 256, 8, 2, 256),
    (1, torch.float8_e4m3fn, 300, 2048, 512, 8, 2, 128),
    (1, torch.bfloat16, 150, 512, 256, 8, 2, 32),    # tile kernel, 32-row blocks
]


@pytest.mark.parametrize("family,wdt,M,K,N,E,k,bm", GATE_UP)
def test_gate_up_sums_are_exact(family, wdt, M, K, N, E, k, bm):
    ids, al, cap, max_blocks = _setup(M, E, k, bm, seed=M + K)
    x = _ints((M, K), -2, 2, 1)
    w13 = _ints((E, 2 * N, K), -2, 2, 2)
    xdt = torch.float32 if (wdt == torch.float32 and family == 0) else \
        (torch.float8_e4m3fn if wdt == torch.float8_e4m3fn else torch.bfloat16)
    one = torch.ones(E, dtype=torch.float32, device=DEV)
    sx = torch.ones(1, dtype=torch.float32, device=DEV)
    hmax = torch.zeros(1, dtype=torch.int32, device=DEV)
    gu = torch.full((cap, 2 * N), float("nan"), dtype=torch.float32, device=DEV)
    probe.gate_up(M, K, N, E, k, bm, max_blocks, _to_dev(x, xdt), _to_dev(w13, wdt),
                  one if wdt == torch.float8_e4m3fn else None, sx, al, hmax, gu, family)
    torch.cuda.synchronize()
    got = gu.cpu().numpy()
    pos = al.pair_pos.cpu().numpy().reshape(M, k)
    for t in range(M):
        for j in range(k):
            want = w13[ids[t, j]] @ x[t]  # [2N] exact integers (gate | up)
            assert np.array_equal(got[pos[t, j]], want.astype(np.float32)), (t, j)


DOWN = [
    (0, torch.bfloat16, 5, 2048, 512, 8, 2, 16),     # expert ring + combine
    (0, torch.bfloat16, 40, 2048, 512, 8, 2, 32),    # ring, 32-column token groups
    (0, torch.float8_e4m3fn, 12, 2048, 1024, 8, 2, 16),
    (0, torch.bfloat16, 2, 2048, 512, 8, 2, 16),     # stream down kernel, combine fused (M < 4)
    (0, torch.float8_e4m3fn, 3, 2048, 1024, 8, 2, 16),
    (1, torch.bfloat16, 200, 2048, 512, 8, 2, 128),  # prefill kernel + combine, 256 x 128
    (1, torch.float8_e4m3fn, 200, 2048, 512, 8, 2, 128),
    (1, torch.bfloat16, 300, 2048, 512, 8, 2, 256),  # 256 x 256 tiles
    (1, torch.float8_e4m3fn, 300, 2048, 1024, 8, 2, 256),
    (1, torch.bfloat16, 150, 1024, 256, 8, 2, 64),   # tile kernel + combine
]


@pytest.mark.parametrize("family,wdt,M,K,N,E,k,bm", DOWN)
def test_down_outputs_are_exact(family, wdt, M, K, N, E, k, bm):
    ids, al, cap, max_blocks = _setup(M, E, k, bm, seed=M + N)
    pos = al.pair_pos.cpu().numpy().reshape(M, k)
    hval = _ints((M, k, N), -2, 2, 3)
    h = np.zeros((cap, N), np.int64)
    for t in range(M):
        for j in range(k):
            h[pos[t, j]] = hval[t, j]
    w2 = _ints((E, K, N), -2, 2, 4)
    hdt = torch.float8_e4m3fn if wdt == torch.float8_e4m3fn else torch.bfloat16
    one = torch.ones(E, dtype=torch.float32, device=DEV)
    sh = torch.ones(1, dtype=torch.float32, device=DEV)
    topk_w = torch.ones(M, k, dtype=torch.float32, device=DEV)
    y = torch.empty(cap, K, dtype=torch.float32, device=DEV)
    out = torch.full((M, K), float("nan"), dtype=torch.float32, device=DEV)
    probe.down(M, K, N, E, k, bm, max_blocks, _to_dev(h, hdt), _to_dev(w2, wdt),
               one if wdt == torch.float8_e4m3fn else None, sh, topk_w, al, y, out, family)
    torch.cuda.synchronize()
    want = np.zeros((M, K), np.int64)
    for t in range(M):
        for j in range(k):
            want[t] += w2[ids[t, j]] @ hval[t, j]
    assert np.abs(want).max() < 2 ** 24
    assert np.array_equal(out.cpu().numpy(), want.astype(np.float32))
