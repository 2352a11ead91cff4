"""Plain CPU oracle of the cache append (numpy, fp64 for the rotation).

TEST INFRASTRUCTURE: only the tests, the smoke check and the bench's CPU
baseline use this module.  It shares nothing with the HIP path.

What it computes, with the passages it follows:

  position      the Sq new tokens of sequence b take positions
                seq_lens[b] - Sq + s (s < Sq): seq_lens already counts them, as
                in the decode module of "DeepSeek MLA 架构详解", which appends the
                new token to both caches and then attends over all of them.
  slot          position t lives at page block_table[b, t // 64], slot t % 64
                (the paged cache with a block table that "DeepSeek-MLA-Principle"
                lists among FlashMLA's ideas, sec. 3).
  RoPE          the rotary embedding of the shared RoPE key (and of the query's
                RoPE part) at the token's position: dimension i < half = d_r / 2
                is paired with dimension i + half (the rotate-half pairing of the
                decode module on the "DeepSeek MLA 架构详解" page), and the pair,
                read as the complex number x_i + j x_{i+half}, is turned by the
                angle pos * 10000^(-i / half), base 10000 ("DeepSeek-MLA-Principle"
                sec. 3, why RoPE: a position-dependent rotation R_pos for which
                <R_m q, R_n k> depends on n - m only).
  e4m3 cache    the pages fix no quantiser.  Per token: amax = max |x| over the
                latent row, s0 = max(amax, 2^-20) / 448 (an fp32 division, the
                precision the kernel decides in), the scale is the smallest power
                of two >= s0 (a per-token power-of-two scale, as in the MX formats
                the hardware converts natively), and r_j = x_j / scale (fp32); the
                code is the E4M3 value nearest to r_j, ties to the even code,
                magnitudes above 448 saturating to 448, sign kept.
  expansion     the values such a cache holds, code * scale, as bf16: the code's
                E4M3 value times the token's scale in one fp32 product, rounded
                to bf16 nearest even (what the bf16 route over an e4m3 cache reads).
"""
from __future__ import annotations

import numpy as np

from . import oracle as O

E4M3_MAX = 448.0
MIN_AMAX = 2.0 ** -20


def positions(seq_lens: np.ndarray, Sq: int) -> np.ndarray:
    """pos[b, s] = seq_lens[b] - Sq + s."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    return seq_lens[:, None] - Sq + np.arange(Sq, dtype=np.int64)[None, :]


def slots(block_table: np.ndarray, seq_lens: np.ndarray, Sq: int):
    """(page, slot) of every new token, each [B, Sq]."""
    pos = positions(seq_lens, Sq)
    bt = np.asarray(block_table, dtype=np.int64)
    page = np.take_along_axis(bt, pos // 64, axis=1)
    return page, pos % 64


def rope(x: np.ndarray, pos) -> np.ndarray:
    """Rotary embedding of the last axis of x (float64) at position pos (a scalar
    or an array broadcasting against x[..., 0]): pair i, the complex number
    x_i + j x_{i+half}, times exp(j pos 10000^(-i/half))."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % 2 == 0, "RoPE needs an even dimension"
    half = d // 2
    angle = np.asarray(pos, dtype=np.float64)[..., None] * np.power(10000.0, -np.arange(half) / half)
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * angle)
    return np.concatenate([z.real, z.imag], axis=-1)


def _e4m3_table() -> np.ndarray:
    """Values of the non-negative finite codes 0x00 .. 0x7E (the oracle's decoder)."""
    L = O.lib()
    return np.array([L.orc_e4m3_value(c) for c in range(0x7F)], dtype=np.float64)


_TABLE = None


def e4m3_nearest(r: np.ndarray) -> np.ndarray:
    """Code of the E4M3 value nearest to each r (float32 array): ties go to the
    even code, magnitudes above 448 saturate, the sign bit follows r's sign."""
    global _TABLE
    if _TABLE is None:
        _TABLE = _e4m3_table()
    r = np.asarray(r, dtype=np.float32)
    a = np.abs(r.astype(np.float64)).reshape(-1)
    dist = np.abs(a[:, None] - _TABLE[None, :])             # [n, 127]
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best                                      # one or two codes (a tie)
    codes = np.arange(0x7F)
    # among the nearest codes prefer an even one (at a tie exactly one is even)
    even_pick = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 0x7F).min(axis=1)
    any_pick = np.where(cand, codes[None, :], 0x7F).min(axis=1)
    mag = np.where(even_pick < 0x7F, even_pick, any_pick)
    sign = np.signbit(r.reshape(-1)).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8).reshape(r.shape)


def quantize_e4m3_rows(x: np.ndarray):
    """Per-row E4M3 quantisation of float32 rows [n, d]: (codes [n, d] uint8,
    scales [n] float32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    s0 = np.maximum(amax, np.float32(MIN_AMAX)).astype(np.float32) / np.float32(E4M3_MAX)
    m, e = np.frexp(s0.astype(np.float64))                    # s0 = m 2^e, m in [0.5, 1)
    scale = np.where(m == 0.5, s0, np.ldexp(1.0, e)).astype(np.float32)
    r = x / scale[..., None]                                 # float32 division
    return e4m3_nearest(r), scale


def expand_e4m3(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """bf16 bits of code * scale for an e4m3 cache (the value semantics of the
    per-token quantisation above): the code's value (the oracle's decoder, sign
    from bit 7) times the token's fp32 scale as one fp32 product, then rounded to
    bf16, nearest even (torch's conversion).  codes [..., d] uint8, scales [...]
    float32 -> uint16 [..., d]."""
    import torch
    codes = np.asarray(codes, dtype=np.uint8)
    mag = _e4m3_table()[np.minimum(codes & 0x7F, 0x7E)].astype(np.float32)   # 0x7F (NaN) never stored
    val = np.where(codes & 0x80, -mag, mag).astype(np.float32)
    prod = (val * np.asarray(scales, dtype=np.float32)[..., None]).astype(np.float32)
    return torch.from_numpy(prod).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def append_kv(c_new, kpe_new, block_table, seq_lens, Sq: int, q_rope=None):
    """Expected effect of appending the new tokens.

    c_new [B, Sq, d_c], kpe_new [B, Sq, d_r] and q_rope [B, Sq, H, d_r] are the
    exact float64 values of the stored inputs.  Returns a dict with
      page, slot  [B, Sq]  where each token is written
      c           [B, Sq, d_c] float64 latent rows (to be stored in the cache dtype)
      codes, scales  [B, Sq, d_c] uint8, [B, Sq] float32 (the e4m3 form of c)
      kpe         [B, Sq, d_r] float64 rotated RoPE keys
      q_rope      [B, Sq, H, d_r] float64 rotated query RoPE parts (None if not given)
    """
    c_new = np.asarray(c_new, dtype=np.float64)
    pos = positions(seq_lens, Sq)
    page, slot = slots(block_table, seq_lens, Sq)
    out = {"page": page, "slot": slot, "pos": pos, "c": c_new}
    codes, scales = quantize_e4m3_rows(c_new.astype(np.float32).reshape(-1, c_new.shape[-1]))
    out["codes"] = codes.reshape(c_new.shape)
    out["scales"] = scales.reshape(c_new.shape[:-1])
    kpe_new = np.asarray(kpe_new, dtype=np.float64)
    out["kpe"] = rope(kpe_new, pos) if kpe_new.shape[-1] > 0 else kpe_new
    if q_rope is not None:
        q = np.asarray(q_rope, dtype=np.float64)
        out["q_rope"] = rope(q, pos[:, :, None])
    else:
        out["q_rope"] = None
    return out
