"""ctypes wrapper around the fp64 CPU oracle (mla_oracle.c).

TEST INFRASTRUCTURE: only the tests, the smoke check and the bench's CPU
baseline use this module.  It imports nothing from the HIP package; its inputs
are the CPU tensors of the seeded generator, in their storage formats.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mla_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16, E4M3, F64 = 0, 1, 2, 3


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Sq", ctypes.c_int32), ("H", ctypes.c_int32),
                ("d_h", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_r", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("scale", ctypes.c_double)]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP over query rows)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        I64 = ctypes.c_int64
        D = ctypes.POINTER(Dims)
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_decode_array.argtypes = [P, I, I64, P]
        L.orc_absorb_q.argtypes = [D, P, I, P, I, P]
        L.orc_decode_splitkv.argtypes = [D, P, I, P, I, P, I, P, P, I, P, P, I, I, P, P]
        L.orc_decode_page_ranges.argtypes = [D, P, I, P, I, P, I, P, P, I, P, P, I, P, P, P, P]
        L.orc_combine_lse.argtypes = [D, I, P, I, P, P, P]
        L.orc_up_v.argtypes = [D, P, I, P, I, P]
        L.orc_decode.argtypes = [D, P, P, I, P, I, P, P, I, P, P, I, P, P, I64, P, P, P, P]
        L.orc_num_threads.restype = I
        _lib = L
    return _lib


def num_threads() -> int:
    return lib().orc_num_threads()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.uint8:
        return E4M3
    if t.dtype == torch.float64:
        return F64
    raise TypeError(t.dtype)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.device.type == "cpu" and t.is_contiguous()
    return ctypes.c_void_p(t.data_ptr())


def _np_ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def dims(B, Sq, H, d_h, d_c, d_r, max_pages, scale, page_size=64) -> Dims:
    return Dims(B, Sq, H, d_h, d_c, d_r, page_size, max_pages, scale)


def dims_of(case) -> Dims:
    wl = case.wl
    return dims(wl.B, wl.Sq, wl.H, wl.d_h, wl.d_c, wl.d_r, case.max_pages, wl.scale)


def decode_values(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a stored tensor (f32 / bf16 / e4m3 codes)."""
    t = t.contiguous()
    out = np.empty(t.numel(), dtype=np.float64)
    lib().orc_decode_array(_p(t), _dt(t), t.numel(), _np_ptr(out))
    return out.reshape(tuple(t.shape))


def cache_values(case) -> np.ndarray:
    """Exact float64 latent cache values (e4m3 code times its token's scale)."""
    c = decode_values(case.c_kv)
    if case.kv_scale is not None:
        c = c * case.kv_scale.double().numpy()[..., None]
    return c


def absorb_q(D: Dims, q_nope: torch.Tensor, W_UK: torch.Tensor) -> np.ndarray:
    out = np.empty((D.B, D.Sq, D.H, D.d_c), dtype=np.float64)
    lib().orc_absorb_q(ctypes.byref(D), _p(q_nope), _dt(q_nope), _p(W_UK), _dt(W_UK),
                       _np_ptr(out))
    return out


def decode_splitkv(D: Dims, q_abs, q_rope, c_kv, kv_scale, k_pe, block_table, seq_lens,
                   num_splits: int, split_pages: int):
    """Split partials: (o_part [B,Sq,H,S,d_c], lse_part [B,Sq,H,S]) in float64."""
    q_abs = q_abs.contiguous()
    o = np.empty((D.B, D.Sq, D.H, num_splits, D.d_c), dtype=np.float64)
    lse = np.empty((D.B, D.Sq, D.H, num_splits), dtype=np.float64)
    ks = None if kv_scale is None else kv_scale.contiguous()
    lib().orc_decode_splitkv(ctypes.byref(D), _p(q_abs), _dt(q_abs), _p(q_rope), _dt(q_rope),
                             _p(c_kv), _dt(c_kv), _p(ks), _p(k_pe), _dt(k_pe),
                             _p(block_table), _p(seq_lens), num_splits, split_pages,
                             _np_ptr(o), _np_ptr(lse))
    return o, lse


def decode_page_ranges(D: Dims, q_abs, q_rope, c_kv, kv_scale, k_pe, block_table, seq_lens,
                       page_begin: np.ndarray, page_end: np.ndarray):
    """Split partials for a split plan given as data: split c of sequence b covers
    its pages [page_begin[b, c], page_end[b, c]).  Returns (o_part, lse_part) in
    float64, shaped as decode_splitkv's."""
    q_abs = q_abs.contiguous()
    pb = np.ascontiguousarray(page_begin, dtype=np.int32)
    pe = np.ascontiguousarray(page_end, dtype=np.int32)
    assert pb.shape == pe.shape and pb.shape[0] == D.B
    S = pb.shape[1]
    o = np.empty((D.B, D.Sq, D.H, S, D.d_c), dtype=np.float64)
    lse = np.empty((D.B, D.Sq, D.H, S), dtype=np.float64)
    ks = None if kv_scale is None else kv_scale.contiguous()
    lib().orc_decode_page_ranges(ctypes.byref(D), _p(q_abs), _dt(q_abs), _p(q_rope), _dt(q_rope),
                                 _p(c_kv), _dt(c_kv), _p(ks), _p(k_pe), _dt(k_pe),
                                 _p(block_table), _p(seq_lens), S, _np_ptr(pb), _np_ptr(pe),
                                 _np_ptr(o), _np_ptr(lse))
    return o, lse


def combine_lse(D: Dims, o_part, lse_part):
    """Log-sum-exp merge. o_part: float64 ndarray or CPU tensor; lse_part float64 ndarray
    or tensor.  Returns (o_latent [B,Sq,H,d_c], lse [B,Sq,H]) in float64."""
    if isinstance(o_part, np.ndarray):
        o_part = torch.from_numpy(np.ascontiguousarray(o_part))
    if isinstance(lse_part, torch.Tensor):
        lse_part = lse_part.double().numpy()
    lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
    S = lse_part.shape[-1]
    o = np.empty((D.B, D.Sq, D.H, D.d_c), dtype=np.float64)
    lse = np.empty((D.B, D.Sq, D.H), dtype=np.float64)
    o_part = o_part.contiguous()
    lib().orc_combine_lse(ctypes.byref(D), S, _p(o_part), _dt(o_part), _np_ptr(lse_part),
                          _np_ptr(o), _np_ptr(lse))
    return o, lse


def up_v(D: Dims, o_latent, W_UV: torch.Tensor) -> np.ndarray:
    if isinstance(o_latent, np.ndarray):
        o_latent = torch.from_numpy(np.ascontiguousarray(o_latent))
    o_latent = o_latent.contiguous()
    out = np.empty((D.B, D.Sq, D.H, D.d_h), dtype=np.float64)
    lib().orc_up_v(ctypes.byref(D), _p(o_latent), _dt(o_latent), _p(W_UV), _dt(W_UV),
                   _np_ptr(out))
    return out


def decode(case, rows: Optional[np.ndarray] = None, D: Optional[Dims] = None):
    """The whole absorbed decode step for selected flat (b,s,h) rows (None = all).

    Returns (out [n,d_h], o_latent [n,d_c], lse [n]) in float64; with rows=None
    the leading axis is reshaped to [B,Sq,H]."""
    D = dims_of(case) if D is None else D
    n_all = D.B * D.Sq * D.H
    r = None
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int64)
    n = n_all if r is None else r.shape[0]
    out = np.empty((n, D.d_h), dtype=np.float64)
    ol = np.empty((n, D.d_c), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    ks = None if case.kv_scale is None else case.kv_scale.contiguous()
    lib().orc_decode(ctypes.byref(D), _p(case.q_nope), _p(case.q_rope), _dt(case.q_nope),
                     _p(case.c_kv), _dt(case.c_kv), _p(ks), _p(case.k_pe), _dt(case.k_pe),
                     _p(case.W_UK), _p(case.W_UV), _dt(case.W_UK),
                     _p(case.block_table), _p(case.seq_lens), n,
                     None if r is None else _np_ptr(r), _np_ptr(out), _np_ptr(ol), _np_ptr(lse))
    if r is None:
        shp = (D.B, D.Sq, D.H)
        return out.reshape(shp + (D.d_h,)), ol.reshape(shp + (D.d_c,)), lse.reshape(shp)
    return out, ol, lse
