"""Seeded synthetic inputs for absorbed-MLA decode.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests.  It holds no arithmetic of the attention method itself: it only draws
random numbers, casts them to storage formats (bf16 round-to-nearest-even,
OCP e4m3 with a per-token scale), and lays them out as a paged cache with a
block table.

Workloads (DeepSeek-V3 dimension table on "DeepSeek-MLA-Principle", section 3;
page size 64 as in the FlashMLA alignment note of "MLA Matrix Absorption",
section 6):

  tiny      B=1   Sq=1 H=8   d_h=32  d_c=64  d_r=16 L=128            fp32, contiguous
  v3_b1     B=1   Sq=1 H=128 d_h=128 d_c=512 d_r=64 L=4096           bf16, identity pages
  v3_b64    B=64  Sq=1 H=128 ...          L ~ U[1024, 8192]          bf16, permuted pages
  v3_long   B=4   Sq=1 H=128 ...          L = 131072                 bf16, permuted pages
  v3_sq4_fp8 B=128 Sq=4 H=128 ...         L ~ U[4096, 16384], causal e4m3 c_kv + fp32 scale

Draw order for a case with numpy ``default_rng(seed)``:
  seq_lens -> page permutation -> c_kv -> k_pe -> q_nope -> q_rope -> W_UK -> W_UV
All draws are float32 standard normal; the weights are multiplied by 0.02.
Unused slots of each sequence's last page hold the finite sentinel 1024.0 so
that an unmasked read cannot go unnoticed.  Unused block-table entries are -1.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

PAGE = 64
SENTINEL = 1024.0
E4M3_MAX = 448.0
# smallest per-token scale: keeps an all-zero row representable
E4M3_MIN_SCALE = 2.0 ** -20


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Sq: int
    H: int
    d_h: int
    d_c: int
    d_r: int
    seq_lo: int           # seq_lens drawn uniform in [seq_lo, seq_hi] (inclusive)
    seq_hi: int
    dtype: str            # "f32" | "bf16" | "fp8"  (storage format of q, W, cache)
    paging: str           # "identity" | "permuted"
    seed: int
    min_splits: int = 1   # the workload asks for at least this many KV chunks per sequence

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_h + self.d_r)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 8, 32, 64, 16, 128, 128, "f32", "identity", 1001),
    "v3_b1": Workload("v3_b1", 1, 1, 128, 128, 512, 64, 4096, 4096, "bf16", "identity", 1002),
    "v3_b64": Workload("v3_b64", 64, 1, 128, 128, 512, 64, 1024, 8192, "bf16", "permuted", 1003),
    "v3_b64_l4096": Workload("v3_b64_l4096", 64, 1, 128, 128, 512, 64, 4096, 4096, "bf16", "permuted", 1006),
    "v3_long": Workload("v3_long", 4, 1, 128, 128, 512, 64, 131072, 131072, "bf16", "permuted",
                        1004, min_splits=32),
    "v3_sq4_fp8": Workload("v3_sq4_fp8", 128, 4, 128, 128, 512, 64, 4096, 16384, "fp8",
                           "permuted", 1005),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (e.g. a smaller B)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


@dataclasses.dataclass
class Case:
    """All inputs of one decode step, as CPU tensors in their storage formats."""
    wl: Workload
    seq_lens: torch.Tensor      # [B] int32
    block_table: torch.Tensor   # [B, max_pages] int32, -1 padded
    c_kv: torch.Tensor          # [P, 64, d_c] f32 | bf16 | uint8 (e4m3 codes)
    kv_scale: Optional[torch.Tensor]  # [P, 64] f32 (fp8 only)
    k_pe: torch.Tensor          # [P, 64, d_r] f32 | bf16
    q_nope: torch.Tensor        # [B, Sq, H, d_h]
    q_rope: torch.Tensor        # [B, Sq, H, d_r]
    W_UK: torch.Tensor          # [H, d_h, d_c]
    W_UV: torch.Tensor          # [H, d_h, d_c]

    @property
    def num_pages(self) -> int:
        return self.c_kv.shape[0]

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.to(torch.int64).sum())


def _to_store(x: np.ndarray, fmt: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if fmt == "f32":
        return t.clone()
    if fmt == "bf16":
        return t.to(torch.bfloat16)          # round-to-nearest-even
    raise ValueError(fmt)


def quantize_e4m3_per_token(x: torch.Tensor):
    """Per-token (last-dim row) OCP e4m3 quantisation of a float32 tensor.

    scale = the smallest power of two >= max(amax, 2^-20) / 448 (the cache format
    the append writes), code = RNE(x / scale) saturated to +-448.
    Returns (uint8 codes, float32 scales with the row shape).
    """
    amax = x.abs().amax(dim=-1)
    s0 = torch.clamp(amax, min=E4M3_MIN_SCALE) / E4M3_MAX
    m, e = torch.frexp(s0)
    scale = torch.where(m == 0.5, s0, torch.ldexp(torch.ones_like(s0), e))
    y = (x / scale.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.to(torch.float32).contiguous()


def draw_seq_lens(rng: np.random.Generator, wl: Workload) -> np.ndarray:
    if wl.seq_lo == wl.seq_hi:
        return np.full(wl.B, wl.seq_lo, dtype=np.int64)
    return rng.integers(wl.seq_lo, wl.seq_hi, size=wl.B, endpoint=True).astype(np.int64)


def make_case(wl: Workload, seed: Optional[int] = None, seq_lens=None,
              max_pages: Optional[int] = None, extra_pages: int = 0) -> Case:
    """Draw every input of one decode step for workload ``wl``.

    ``seq_lens`` overrides the drawn lengths (the draw still happens, so the
    remaining streams are unchanged).  ``max_pages`` widens the block table.
    ``extra_pages`` appends never-referenced sentinel pages to the cache.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    drawn = draw_seq_lens(rng, wl)
    lens = drawn if seq_lens is None else np.asarray(seq_lens, dtype=np.int64)
    assert lens.shape == (wl.B,)
    pages_per_seq = (lens + PAGE - 1) // PAGE
    total_pages = int(pages_per_seq.sum())
    P = total_pages + extra_pages
    if wl.paging == "identity":
        perm = np.arange(total_pages)
        rng.permutation(max(total_pages, 1))   # keep the stream aligned with "permuted"
    else:
        perm = rng.permutation(total_pages)
    mp = int(pages_per_seq.max()) if wl.B > 0 else 0
    mp = max(mp, 1) if max_pages is None else max_pages
    assert mp >= int(pages_per_seq.max(initial=0))
    bt = np.full((wl.B, mp), -1, dtype=np.int32)
    off = 0
    for b in range(wl.B):
        n = int(pages_per_seq[b])
        bt[b, :n] = perm[off:off + n]
        off += n

    # cache rows, drawn in physical page order
    c32 = rng.standard_normal((P, PAGE, wl.d_c), dtype=np.float32)
    r32 = rng.standard_normal((P, PAGE, wl.d_r), dtype=np.float32)
    # sentinel in the unused tail slots of each last page and in unreferenced pages
    for b in range(wl.B):
        n = int(lens[b])
        if n % PAGE and n > 0:
            p = bt[b, n // PAGE]
            c32[p, n % PAGE:, :] = SENTINEL
            r32[p, n % PAGE:, :] = SENTINEL
    if extra_pages:
        c32[total_pages:] = SENTINEL
        r32[total_pages:] = SENTINEL
    qn = rng.standard_normal((wl.B, wl.Sq, wl.H, wl.d_h), dtype=np.float32)
    qr = rng.standard_normal((wl.B, wl.Sq, wl.H, wl.d_r), dtype=np.float32)
    wuk = rng.standard_normal((wl.H, wl.d_h, wl.d_c), dtype=np.float32) * np.float32(0.02)
    wuv = rng.standard_normal((wl.H, wl.d_h, wl.d_c), dtype=np.float32) * np.float32(0.02)

    wfmt = "f32" if wl.dtype == "f32" else "bf16"
    kv_scale = None
    if wl.dtype == "fp8":
        codes, kv_scale = quantize_e4m3_per_token(torch.from_numpy(c32))
        # sentinel slots: code 0x7E (448) with scale 1024/448 decodes to 1024
        for b in range(wl.B):
            n = int(lens[b])
            if n % PAGE and n > 0:
                p = bt[b, n // PAGE]
                codes[p, n % PAGE:, :] = 0x7E
                kv_scale[p, n % PAGE:] = SENTINEL / E4M3_MAX
        if extra_pages:
            codes[total_pages:] = 0x7E
            kv_scale[total_pages:] = SENTINEL / E4M3_MAX
        c_kv = codes
    else:
        c_kv = _to_store(c32, wfmt)
    del c32
    return Case(
        wl=wl,
        seq_lens=torch.from_numpy(lens.astype(np.int32)),
        block_table=torch.from_numpy(bt),
        c_kv=c_kv,
        kv_scale=kv_scale,
        k_pe=_to_store(r32, wfmt),
        q_nope=_to_store(qn, wfmt),
        q_rope=_to_store(qr, wfmt),
        W_UK=_to_store(wuk, wfmt),
        W_UV=_to_store(wuv, wfmt),
    )


# --- stand-alone inputs for testing one entry point in isolation ------------

def latent_format(wl: Workload) -> str:
    """Storage format of the absorbed query and of the merged latent output."""
    return "f32" if wl.dtype == "f32" else "bf16"


def random_q_abs(wl: Workload, seed: int) -> torch.Tensor:
    """An absorbed query with the spread the product q_nope . W_UK would have:
    entries ~ N(0, d_h * 0.02^2)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((wl.B, wl.Sq, wl.H, wl.d_c), dtype=np.float32)
    x *= np.float32(math.sqrt(wl.d_h) * 0.02)
    return _to_store(x, latent_format(wl))


def random_partials(wl: Workload, num_splits: int, seed: int, empty_frac: float = 0.25):
    """Random split partials: o_part [B,Sq,H,S,d_c] f32, lse_part [B,Sq,H,S] f32,
    with a fraction of the splits marked empty (lse = -inf, o = NaN garbage) and
    at least one non-empty split per row."""
    rng = np.random.default_rng(seed)
    shp = (wl.B, wl.Sq, wl.H, num_splits)
    o = rng.standard_normal(shp + (wl.d_c,), dtype=np.float32)
    lse = (rng.standard_normal(shp, dtype=np.float32) * np.float32(4.0) + np.float32(6.0))
    empty = rng.random(shp) < empty_frac
    empty[..., 0] = False
    lse[empty] = -np.inf
    o[empty] = np.nan      # an empty split's o is unspecified; NaN makes a read visible
    return torch.from_numpy(o), torch.from_numpy(lse)


def random_o_latent(wl: Workload, seed: int) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((wl.B, wl.Sq, wl.H, wl.d_c), dtype=np.float32)
    return _to_store(x, latent_format(wl))


def random_new_tokens(wl: Workload, seed: int, fmt: Optional[str] = None, latent_std: float = 3.0):
    """The new tokens' latent rows [B, Sq, d_c] and un-rotated RoPE keys
    [B, Sq, d_r] of an append (normal; latent rows with standard deviation
    ``latent_std``, 3 by default so that the per-token e4m3 scales vary), stored
    as ``fmt`` (default: the workload's activation format)."""
    rng = np.random.default_rng(seed)
    c = rng.standard_normal((wl.B, wl.Sq, wl.d_c), dtype=np.float32) * np.float32(latent_std)
    r = rng.standard_normal((wl.B, wl.Sq, wl.d_r), dtype=np.float32)
    fmt = fmt or ("f32" if wl.dtype == "f32" else "bf16")
    return _to_store(c, fmt), _to_store(r, fmt)
