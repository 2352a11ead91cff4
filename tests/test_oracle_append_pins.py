"""Pins of the cache-append oracle (oracle/append.py) against what the pages
and the mathematics fix, not against itself:

  * RoPE: identity at position 0; the complex-number form of a rotation by
    pos * 10000^(-i/half) (an independent formula); the relative-position
    property <R_m q, R_n k> = <q, R_{n-m} k> that "DeepSeek-MLA-Principle"
    sec. 3 (why RoPE) states; composition of rotations; hand-computed values
    that fix the frequency schedule;
  * the E4M3 quantiser: torch's float8_e4m3fn conversion (a library routine) on
    random values and on every exact midpoint between codes, the OCP maximum,
    and the per-token scale on rows whose amax is a power of two times 448;
  * placement: positions and slots of a hand-built block table.
"""
import math

import numpy as np
import pytest
import torch

from oracle import append as A


def test_rope_identity_at_position_zero():
    x = np.random.default_rng(0).standard_normal((5, 64))
    assert np.array_equal(A.rope(x, 0), x)


@pytest.mark.parametrize("d", [2, 8, 64])
def test_rope_is_complex_rotation(d):
    """Pair (x_i, x_{i+half}) as the complex number x_i + j x_{i+half}, multiplied
    by exp(j pos 10000^(-i/half))."""
    rng = np.random.default_rng(d)
    x = rng.standard_normal((3, d))
    half = d // 2
    for pos in (1, 7, 4095, 131071):
        z = x[:, :half] + 1j * x[:, half:]
        w = np.exp(1j * pos * np.power(10000.0, -np.arange(half) / half))
        zr = z * w
        y = A.rope(x, pos)
        np.testing.assert_allclose(y[:, :half], zr.real, rtol=0, atol=1e-9)
        np.testing.assert_allclose(y[:, half:], zr.imag, rtol=0, atol=1e-9)


def test_rope_relative_position_property():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in ((0, 5), (3, 3), (100, 37), (4096, 8191), (70000, 131071)):
        lhs = A.rope(q, m) @ A.rope(k, n)
        rhs = q @ A.rope(k, n - m)
        assert abs(lhs - rhs) <= 1e-9 * (np.linalg.norm(q) * np.linalg.norm(k))


def test_rope_composes_and_preserves_pair_norms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 64))
    np.testing.assert_allclose(A.rope(A.rope(x, 123), 456), A.rope(x, 579), rtol=0, atol=1e-9)
    y = A.rope(x, 999)
    np.testing.assert_allclose(np.hypot(y[:, :32], y[:, 32:]), np.hypot(x[:, :32], x[:, 32:]), rtol=1e-13)


def test_rope_hand_values():
    # d = 2: the only frequency is 1, so position p rotates by p radians
    y = A.rope(np.array([1.0, 0.0]), 1)
    assert y[0] == pytest.approx(math.cos(1.0), abs=1e-15) and y[1] == pytest.approx(math.sin(1.0), abs=1e-15)
    # d = 4: pair i = 1 has frequency 10000^(-1/2) = 0.01, so position 100 rotates it by 1 radian
    y = A.rope(np.array([0.0, 1.0, 0.0, 0.0]), 100)
    np.testing.assert_allclose(y, [0.0, math.cos(1.0), 0.0, math.sin(1.0)], atol=1e-12)
    # d = 64: pair i = 16 has frequency 10000^(-1/2); the rotation is by pos/100 radians
    x = np.zeros(64)
    x[16] = 2.0
    y = A.rope(x, 250)
    assert y[16] == pytest.approx(2.0 * math.cos(2.5), abs=1e-12)
    assert y[48] == pytest.approx(2.0 * math.sin(2.5), abs=1e-12)


def _torch_e4m3(r: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.clip(np.asarray(r, np.float32), -448, 448))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_nearest_matches_library_conversion():
    table = A._e4m3_table()
    mids = ((table[1:] + table[:-1]) / 2).astype(np.float32)       # exact in fp32: every tie
    rng = np.random.default_rng(3)
    r = np.concatenate([mids, -mids, rng.standard_normal(20000).astype(np.float32) * 60,
                        (rng.standard_normal(2000) * 2.0 ** -8).astype(np.float32),
                        np.array([0.0, -0.0, 448.0, -448.0, 460.0, 470.0, 1e6, -1e6], np.float32)])
    assert np.array_equal(A.e4m3_nearest(r), _torch_e4m3(r))


def test_e4m3_quantise_rows():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 512)).astype(np.float32)
    x[1] *= 1e-9                               # amax below 2^-20: scale floored
    x[2, 7] = 448.0 * 4                        # amax 1792: scale exactly 4, the max maps to 0x7E
    codes, scales = A.quantize_e4m3_rows(x)
    assert scales.dtype == np.float32
    assert scales[2] == np.float32(4.0) and codes[2, 7] == 0x7E
    assert scales[1] == np.float32(2.0 ** -20) / np.float32(448.0)
    for i in range(6):
        amax = np.float32(max(np.abs(x[i]).max(), np.float32(2.0 ** -20)))
        s = amax / np.float32(448.0)
        assert scales[i] == s
        assert np.array_equal(codes[i], _torch_e4m3(x[i] / s))


def test_positions_and_slots():
    bt = np.array([[5, 9, 2, -1], [7, 3, -1, -1]], dtype=np.int32)
    seq_lens = np.array([130, 66], dtype=np.int32)
    page, slot = A.slots(bt, seq_lens, Sq=4)
    # sequence 0: positions 126..129 -> pages 9, 9, 2, 2; slots 62, 63, 0, 1
    assert page[0].tolist() == [9, 9, 2, 2] and slot[0].tolist() == [62, 63, 0, 1]
    # sequence 1: positions 62..65 -> pages 7, 7, 3, 3
    assert page[1].tolist() == [7, 7, 3, 3] and slot[1].tolist() == [62, 63, 0, 1]
    assert A.positions(seq_lens, 4)[1].tolist() == [62, 63, 64, 65]


def test_expand_is_decoded_code_times_scale():
    """The expansion of an e4m3 cache: with a power-of-two scale the product is
    exact, so the bf16 value equals the code's OCP value times the scale (every
    e4m3 value has at most 4 significant bits, exact in bf16); with other scales it
    is the fp32 product rounded to bf16."""
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F].reshape(1, -1)            # no NaN codes
    for sc in (1.0, 2.0 ** -9, 16.0):
        got = A.expand_e4m3(codes, np.array([sc], np.float32))
        vals = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).double().numpy()[0]
        ref = torch.from_numpy(codes[0].copy()).view(torch.float8_e4m3fn).double().numpy() * sc
        assert np.array_equal(vals, ref)
    sc = np.float32(0.3)
    got = A.expand_e4m3(codes, np.array([sc], np.float32))
    ref = (torch.from_numpy(codes[0].copy()).view(torch.float8_e4m3fn).float() * torch.tensor(0.3)).bfloat16()
    assert np.array_equal(got[0], ref.view(torch.int16).numpy().view(np.uint16))
