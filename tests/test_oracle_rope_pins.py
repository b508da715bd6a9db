"""Pins of the oracle's rotary embedding + per-head E4M3 quantisation
(oracle_rope_quant_per_head) against what mathematics and library routines
fix, independently of the oracle's own loops: the zero angle is the identity
and reduces to the pinned per-tensor quantiser per head; the rotation equals
a complex multiplication by exp(i a) (numpy's complex arithmetic) for both
pairings; it preserves pair norms and depends only on position differences
in inner products; the inverse flag is the rotation at negated positions and
undoes the forward one; the codes equal torch's E4M3 cast of the clamped
quotient; the largest element of each head gets the largest code."""
import numpy as np
import pytest
import torch

import oracle
from tests import bruteforce as bf


def _case(T=7, nH=3, D=16, seed=0, dtype=np.float32, pos=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, nH, D)).astype(np.float32)
    if dtype == np.uint16:  # bf16 bits
        x = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if pos is None:
        pos = rng.integers(0, 4096, size=T).astype(np.int32)
    invf = (10000.0 ** (-np.arange(0, D, 2) / D)).astype(np.float32)
    return x, pos, invf


def _angles(pos, invf):
    return (pos.astype(np.float64)[:, None] * invf.astype(np.float64)[None, :]).astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_zero_positions_are_the_identity_and_per_head_per_tensor_quantisation(dtype):
    x, _, invf = _case(dtype=dtype)
    T, nH, D = x.shape
    codes, scales, y = oracle.rope_quant_per_head(x, np.zeros(T, np.int32), invf, want_y=True)
    assert np.array_equal(y, bf.decode(x))
    for h in range(nH):
        xh = np.ascontiguousarray(x[:, h, :])
        s = oracle.act_scale(xh)
        assert scales[h] == np.float32(s)
        assert np.array_equal(codes[:, h, :], oracle.quantize_e4m3(xh, s))


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_is_a_complex_multiplication(interleaved):
    x, pos, invf = _case(T=11, nH=4, D=32, seed=3)
    _, _, y = oracle.rope_quant_per_head(x, pos, invf, interleaved=interleaved, want_y=True)
    a = _angles(pos, invf)[:, None, :]
    xd = x.astype(np.float64)
    if interleaved:
        z = (xd[..., 0::2] + 1j * xd[..., 1::2]) * np.exp(1j * a)
        ref = np.empty_like(xd)
        ref[..., 0::2], ref[..., 1::2] = z.real, z.imag
    else:
        h = x.shape[2] // 2
        z = (xd[..., :h] + 1j * xd[..., h:]) * np.exp(1j * a)
        ref = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)
    # pair norms preserved
    if interleaved:
        n0 = xd[..., 0::2] ** 2 + xd[..., 1::2] ** 2
        n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    else:
        h = x.shape[2] // 2
        n0 = xd[..., :h] ** 2 + xd[..., h:] ** 2
        n1 = y[..., :h] ** 2 + y[..., h:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)


def test_unit_pair_rotates_counter_clockwise():
    """x = (1, 0) in pair 0 (halves pairing: elements 0 and D/2) at angle a
    becomes (cos a, sin a); at -a (inverse) (cos a, -sin a)."""
    D = 4
    x = np.zeros((1, 1, D), np.float32)
    x[0, 0, 0] = 1.0
    invf = np.array([0.5, 0.25], np.float32)
    pos = np.array([3], np.int32)  # a = 1.5 exactly
    _, _, y = oracle.rope_quant_per_head(x, pos, invf, want_y=True)
    assert (y[0, 0, 0], y[0, 0, 2]) == (np.cos(1.5), np.sin(1.5))
    assert y[0, 0, 1] == 0.0 and y[0, 0, 3] == 0.0
    _, _, yi = oracle.rope_quant_per_head(x, pos, invf, inverse=True, want_y=True)
    assert (yi[0, 0, 0], yi[0, 0, 2]) == (np.cos(1.5), -np.sin(1.5))


@pytest.mark.parametrize("interleaved", [False, True])
def test_inverse_is_negated_positions_and_undoes_the_rotation(interleaved):
    x, pos, invf = _case(T=9, nH=2, D=16, seed=5)
    c1, s1, y1 = oracle.rope_quant_per_head(x, pos, invf, interleaved, inverse=True, want_y=True)
    c2, s2, y2 = oracle.rope_quant_per_head(x, -pos, invf, interleaved, inverse=False, want_y=True)
    assert np.array_equal(y1, y2) and np.array_equal(c1, c2) and np.array_equal(s1, s2)
    _, _, y = oracle.rope_quant_per_head(x, pos, invf, interleaved, want_y=True)
    _, _, back = oracle.rope_quant_per_head(y.astype(np.float32), pos, invf, interleaved,
                                            inverse=True, want_y=True)
    np.testing.assert_allclose(back, x.astype(np.float64), rtol=0, atol=4e-7 * np.abs(x).max())


def test_inner_products_depend_only_on_position_differences():
    """<R(p) q, R(p') k> is a function of p - p' (both rotated with the same
    frequencies).  The angles are fl32(pos * inv_freq), each within 2^-24 of
    its exact value relative, so at positions below 40 the products agree to
    2 * 40 * 2^-24 * sum|q||k| / |<q, k>|, well inside 1e-5 here."""
    rng = np.random.default_rng(8)
    D = 32
    qk = rng.standard_normal((2, 1, D)).astype(np.float32)
    invf = (10000.0 ** (-np.arange(0, D, 2) / D)).astype(np.float32)
    vals = []
    for shift in (0, 5, 17):
        pos = np.array([3 + shift, 11 + shift], np.int32)
        _, _, y = oracle.rope_quant_per_head(qk, pos, invf, want_y=True)
        vals.append(float(y[0, 0] @ y[1, 0]))
    np.testing.assert_allclose(vals, vals[0], rtol=1e-5)


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_codes_are_the_torch_cast_of_the_clamped_quotient(dtype):
    x, pos, invf = _case(T=13, nH=5, D=32, seed=9, dtype=dtype)
    codes, scales, y = oracle.rope_quant_per_head(x, pos, invf, want_y=True)
    amax = np.abs(y).max(axis=(0, 2))
    assert np.array_equal(scales, (amax / 448.0).astype(np.float32))
    q = (y / scales.astype(np.float64)[None, :, None]).astype(np.float32)
    ref = bf.e4m3_cast(q)
    assert np.array_equal(bf.decode(codes), ref)
    for h in range(x.shape[1]):
        t, d = np.unravel_index(np.argmax(np.abs(y[:, h, :])), y[:, h, :].shape)
        assert codes[t, h, d] & 0x7F == 0x7E


def test_static_scales_and_zero_heads():
    x, pos, invf = _case(T=4, nH=3, D=8, seed=11)
    x[:, 1, :] = 0.0
    codes, scales = oracle.rope_quant_per_head(x, pos, invf)
    assert scales[1] == 1.0 and not (codes[:, 1, :] & 0x7F).any()  # +-0
    st = np.array([0.5, 0.25, 0.001], np.float32)
    codes2, scales2, y = oracle.rope_quant_per_head(x, pos, invf, static_scales=st, want_y=True)
    assert np.array_equal(scales2, st)
    # a tiny static scale saturates: every |y| / s >= 448 of head 2 gets +-448
    big = np.abs(y[:, 2, :]) / np.float64(st[2]) >= 448.0
    assert big.sum() > 10 and np.all((codes2[:, 2, :][big] & 0x7F) == 0x7E)
