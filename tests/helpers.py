"""Shared plumbing for the test suite: parameter structs for a generated case,
copying a case to the GPU, the error metric, and row sampling."""
from __future__ import annotations

import bisect

import numpy as np
import torch

from mla_latent_kv_05_amd import inputs as I
from mla_latent_kv_05_amd import mla

# max|gpu - oracle| / RMS(oracle): fp32 inputs, bf16 inputs, fp8 latent cache
TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


def err_rms(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(got - ref))) / rms


def err_rows(got, ref, out_bf16=False) -> float:
    """max over rows (last axis) of max|got - ref| / RMS(ref row); rows whose reference
    is 0 (nothing visible) must be 0 exactly.  For many new tokens per sequence: the
    rows see from one position to thousands, and a row that sees few positions
    returns a few value rows at their full size, while the whole-output RMS is set
    by the rows that average many positions.  With a bf16 output, each element's own
    rounding (at most 2^-9 of its value; 2^-8 allowed) is taken off first."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(got.shape)
    rms = np.sqrt(np.mean(ref ** 2, axis=1))
    empty = rms == 0
    assert (got[empty] == 0).all()
    d = np.abs(got - ref)
    if out_bf16:
        d = np.maximum(d - 2.0 ** -8 * np.abs(ref), 0.0)
    return float((d.max(axis=1)[~empty] / rms[~empty]).max())


def assert_bf16_rounding(got, ref, acc_rel=1e-3):
    """Every element is within half a bf16 ulp (at most 2^-8 relative) of the exact
    value, plus an accumulation allowance of acc_rel * RMS(ref)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bound = np.abs(ref) * 2.0 ** -8 + acc_rel * rms
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{int(bad.sum())} elements beyond bf16 rounding, worst excess " \
        f"{float(np.max(np.abs(got - ref) - bound)):.3e}"


# start cost of a sequence in the balanced plan's work units (the C header's num_parts)
SEQ_START_COST = 6


def split_page_ranges(seq_lens, p: mla.Params):
    """Pages [begin, end) of sequence b that split slot c covers under p's split plan,
    as two [B, num_splits] int32 arrays (end <= begin: empty).  Written from the
    plan's definition in the C header, independently of the kernels: fixed splits
    cover [c*split_pages, (c+1)*split_pages); balanced splits give a sequence of
    n > 0 pages SEQ_START_COST + n work units (start cost first, then one per page),
    cut the batch's units, taken in sequence order, into num_parts parts at
    floor(j*U/P), and slot c of sequence b is its share of the pages of the (c+1)-th
    part that holds any of them."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    n = (lens + 63) // 64
    B, S = len(lens), p.num_splits
    beg = np.zeros((B, S), np.int64)
    end = np.zeros((B, S), np.int64)
    if p.num_parts == 0:
        for b in range(B):
            for c in range(S):
                beg[b, c] = c * p.split_pages
                end[b, c] = min((c + 1) * p.split_pages, n[b])
        return beg.astype(np.int32), np.maximum(end, beg).astype(np.int32)
    cost = np.where(n > 0, n + SEQ_START_COST, 0)
    P, U = p.num_parts, int(cost.sum())
    starts = [j * U // P for j in range(P + 1)]
    off = 0
    for b in range(B):
        if n[b] > 0:
            first = off + SEQ_START_COST           # unit of the sequence's first page
            # the parts holding the sequence's first and last pages
            j0 = bisect.bisect_right(starts[:P], first) - 1
            jl = bisect.bisect_right(starts[:P], first + n[b] - 1) - 1
            for j in range(j0, jl + 1):
                c = j - j0
                assert c < S, f"sequence {b} touches more than num_splits={S} parts"
                beg[b, c] = max(starts[j] - first, 0)
                end[b, c] = min(starts[j + 1] - first, n[b])
        off += cost[b]
    return beg.astype(np.int32), np.maximum(end, beg).astype(np.int32)


def params_for(case: I.Case, num_splits=None, split_pages=None, flags=0, out_dtype=None,
               plan=False, num_cus=256, num_parts=0, part_dtype=None) -> mla.Params:
    """Parameters for a case.  bench=True-like use: plan=True with part_dtype=mla.BF16
    is the launch configuration the bench times for bf16 and e4m3 caches."""
    wl = case.wl
    f32 = wl.dtype == "f32"
    fl = mla.F32 if f32 else mla.BF16
    kv = mla.FP8_E4M3 if wl.dtype == "fp8" else fl
    if num_parts:
        # balanced splits with exactly as many slots as the plan needs (+ extra_slots)
        num_splits, split_pages = 1, 1
    elif num_splits is None and split_pages is None:
        num_splits = 1
    if num_splits is None:
        num_splits = -(-case.max_pages // split_pages)
    p = mla.make_params(wl.B, wl.Sq, wl.H, wl.d_h, wl.d_c, wl.d_r, case.num_pages, case.max_pages,
                        num_splits=num_splits, split_pages=split_pages, scale=wl.scale,
                        q_dtype=fl, w_dtype=fl, kv_dtype=kv, pe_dtype=fl, latent_dtype=fl,
                        out_dtype=mla.F32 if out_dtype is None else out_dtype, flags=flags,
                        num_parts=num_parts, part_dtype=mla.F32 if part_dtype is None else part_dtype)
    if num_parts:
        p.num_splits = max(1, int(touched_parts(case.seq_lens, num_parts).max()))
    if plan:
        p = mla.plan_splits(p, int(case.seq_lens.max()), case.total_tokens, num_cus=num_cus,
                            min_splits=wl.min_splits)
    return p


class DeviceCase:
    """The tensors of a Case on the GPU (storage formats unchanged)."""

    def __init__(self, case: I.Case, device="cuda"):
        self.case = case
        for f in ("seq_lens", "block_table", "c_kv", "k_pe", "q_nope", "q_rope", "W_UK", "W_UV"):
            setattr(self, f, getattr(case, f).to(device).contiguous())
        self.kv_scale = None if case.kv_scale is None else case.kv_scale.to(device).contiguous()

    def step(self, p: mla.Params) -> mla.DecodeStep:
        st = mla.DecodeStep(p)
        st(self.q_nope, self.q_rope, self.c_kv, self.k_pe, self.kv_scale, self.block_table,
           self.seq_lens, self.W_UK, self.W_UV)
        return st


def sample_rows(case: I.Case, n_seq: int, heads_per_seq: int, seed: int = 0) -> np.ndarray:
    """Flat (b,s,h) rows: the shortest and longest sequences plus random ones, every
    query row s, a spread of heads (first, last, random)."""
    wl = case.wl
    rng = np.random.default_rng(seed)
    lens = case.seq_lens.numpy()
    seqs = {int(lens.argmin()), int(lens.argmax())}
    while len(seqs) < min(n_seq, wl.B):
        seqs.add(int(rng.integers(wl.B)))
    heads = {0, wl.H - 1}
    while len(heads) < min(heads_per_seq, wl.H):
        heads.add(int(rng.integers(wl.H)))
    rows = [(b * wl.Sq + s) * wl.H + h for b in sorted(seqs) for s in range(wl.Sq) for h in sorted(heads)]
    return np.array(rows, dtype=np.int64)


def touched_parts(seq_lens, num_parts: int) -> np.ndarray:
    """Number of balanced-split parts holding pages of each sequence (0 for an empty one)."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    n = (lens + 63) // 64
    cost = np.where(n > 0, n + SEQ_START_COST, 0)
    U, P = int(cost.sum()), num_parts
    starts = [j * U // P for j in range(P)]
    off = np.concatenate([[0], np.cumsum(cost)[:-1]])
    out = np.zeros(len(n), np.int64)
    for b in range(len(n)):
        if n[b]:
            first = off[b] + SEQ_START_COST
            out[b] = (bisect.bisect_right(starts, first + n[b] - 1) - bisect.bisect_right(starts, first)) + 1
    return out
