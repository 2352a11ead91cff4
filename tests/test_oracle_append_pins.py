"""Pins of the cache-append oracle (oracle/append.py) against what the pages
and the mathematics fix, not against itself:

  * RoPE: identity at position 0; the real 2 x 2 rotation matrix of each pair
    at angle pos / 10000^(i/half) (an independent form); the relative-position
    property <R_m q, R_n k> = <q, R_{n-m} k> that "DeepSeek-MLA-Principle"
    sec. 3 (why RoPE) states; composition of rotations; hand-computed values
    that fix the frequency schedule;
  * the E4M3 quantiser: torch's float8_e4m3fn conversion (a library routine) on
    random values and on every exact midpoint between codes, the OCP maximum,
    and the per-token scale: the smallest power of two at or above
    max(amax, 2^-20) / 448, checked by its defining inequalities and on rows
    whose amax is a power of two times 448;
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
def test_rope_is_a_plane_rotation_per_pair(d):
    """Each pair (x_i, x_{i+half}) is multiplied by the 2 x 2 rotation matrix
    [[cos a, -sin a], [sin a, cos a]] with a = pos * base^(-i/half), the angle
    taken as pos / base^(i/half) (and the frequencies from math, not numpy)."""
    rng = np.random.default_rng(d)
    x = rng.standard_normal((3, d))
    half = d // 2
    for pos in (1, 7, 4095, 131071):
        y = A.rope(x, pos)
        for i in range(half):
            a = pos / (10000.0 ** (i / half))
            rot = np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]])
            pair = rot @ np.stack([x[:, i], x[:, i + half]])
            np.testing.assert_allclose(y[:, i], pair[0], rtol=0, atol=1e-9)
            np.testing.assert_allclose(y[:, i + half], pair[1], rtol=0, atol=1e-9)


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
    x[3, 0] = 448.0 * 4 * 1.0000001           # just above: the next power of two
    codes, scales = A.quantize_e4m3_rows(x)
    assert scales.dtype == np.float32
    assert scales[2] == np.float32(4.0) and codes[2, 7] == 0x7E
    assert scales[3] == np.float32(8.0)
    # 2^-20 / 448 = 2^-28 / 1.75: the scale of a floored row is 2^-28
    assert scales[1] == np.float32(2.0 ** -28)
    for i in range(6):
        amax = np.float32(max(np.abs(x[i]).max(), np.float32(2.0 ** -20)))
        s0 = amax / np.float32(448.0)
        s = float(scales[i])
        assert math.frexp(s)[0] == 0.5                   # a power of two
        assert s >= float(s0) and s / 2 < float(s0)      # the smallest one >= s0
        assert np.array_equal(codes[i], _torch_e4m3(x[i] / np.float32(s)))


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


def _round_sig(x, bits):
    """x (float64, normal range or 0) rounded to `bits` significant bits, ties to
    even: frexp gives x = m * 2^e with 0.5 <= |m| < 1, so m * 2^bits is exact and
    rint rounds it to the nearest integer, halves to even."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(m * 2.0 ** bits), e - bits)


def _bf16_bits_value(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def test_expand_rounds_the_fp32_product_to_bf16():
    """Expansion = the code's value times the scale as one fp32 product (24
    significant bits), then bf16 (8 significant bits), each nearest-even, written
    here from the two formats' significand widths.  The case list includes
    products for which rounding the exact product straight to bf16 gives another
    value (the fp32 product lands exactly on a bf16 midpoint), so a single
    rounding would fail this pin."""
    rng = np.random.default_rng(31)
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]                           # no NaN codes
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    # random scales that are not powers of two
    scales = (rng.uniform(1e-3, 8.0, size=400)).astype(np.float32)
    scales = scales[np.frexp(scales.astype(np.float64))[0] != 0.5]
    # constructed scales: v * s exact lies just above a bf16 midpoint that is an fp32 value
    built = []
    for v in (1.125, 1.375, 1.625, 1.875, 3.0, 5.0, 7.0, 0.4375, 13.0):
        for mant in range(128, 256, 2):                           # even bf16 significands
            mid = (mant + 0.5) * 2.0 ** -7                        # midpoint above it, in [1, 2)
            s0 = np.float32(mid / v)
            for k in range(-4, 5):
                s = np.nextafter(s0, np.float32(np.inf) if k > 0 else np.float32(0), dtype=np.float32)
                for _ in range(abs(k) - 1):
                    s = np.nextafter(s, np.float32(np.inf) if k > 0 else np.float32(0), dtype=np.float32)
                s = s0 if k == 0 else s
                p = v * float(s)                                  # exact: 4 x 24 bits
                if _round_sig(p, 24) == mid and p != mid:
                    built.append(s)
    built = np.unique(np.array(built, dtype=np.float32))
    assert built.size >= 50
    all_scales = np.concatenate([scales, built])
    got = A.expand_e4m3(np.broadcast_to(codes, (all_scales.size, codes.size)).copy(), all_scales)
    exact = vals[None, :] * all_scales.astype(np.float64)[:, None]   # exact products
    ref = _round_sig(_round_sig(exact, 24), 8)
    assert np.array_equal(_bf16_bits_value(got), ref)
    # the constructed cases tell the two roundings apart
    once = _round_sig(exact, 8)
    assert int((once != ref).sum()) >= 50
