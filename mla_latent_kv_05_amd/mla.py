"""ctypes binding of libmla.so (include/mla.h), same entry-point names.

Argument marshalling only: tensors must already be on the GPU, contiguous and
in the dtypes the parameters declare; every step of the computation runs in
the library's HIP kernels.  Torch provides device memory and the stream.
There is no CPU fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla.so")
DEBUG_LIB_PATH = os.path.join(PKG, "libmla_debug.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
FLAG_GENERIC = 1
FLAG_ROWS64 = 2       # force the eight-wave 64-row attention kernel (bf16 cache)
FLAG_ROWS128 = 4      # force the four-wave 128-row attention kernel
FLAG_POW2_SCALE = 8   # e4m3 cache: every kv_scale is a power of two (as mla_append_kv writes)
PAGE = 64

STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_DTYPE",
          4: "MLA_ERR_SPLITS", 5: "MLA_ERR_HIP", 6: "MLA_ERR_UNSUPPORTED"}

# every symbol include/mla.h declares
EXPORTS = ("mla_absorb_q", "mla_decode_splitkv", "mla_combine_lse", "mla_up_v", "mla_combine_up_v",
           "mla_append_kv", "mla_decompress_kv", "mla_prefill_attention", "mla_prefer_absorbed", "mla_prefill_lmax", "mla_expand_kv",
           "mla_decode_step", "mla_decode_step_workspace", "mla_decode_step_noalloc",
           "mla_decode_step_persistent", "mla_decode_step_persistent_workspace",
           "mla_device_errors", "mla_debug_bounds",
           "mla_check_params", "mla_plan_splits", "mla_default_num_splits", "mla_decode_kernel_name",
           "mla_status_string", "mla_last_error", "mla_abi_version")


class MLAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Params(ctypes.Structure):
    """mirror of mla_params_t"""
    _fields_ = [("B", ctypes.c_int32), ("Sq", ctypes.c_int32), ("H", ctypes.c_int32),
                ("d_h", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_r", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("split_pages", ctypes.c_int32), ("scale", ctypes.c_float),
                ("q_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("pe_dtype", ctypes.c_int32),
                ("latent_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("num_parts", ctypes.c_int32), ("part_dtype", ctypes.c_int32)]

    def copy(self) -> "Params":
        q = Params()
        ctypes.pointer(q)[0] = self
        return q

    def __repr__(self):
        return "Params(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_lib = None
_debug_lib = None


def lib():
    """Load libmla.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def debug_lib():
    """libmla_debug.so (built with the MLA_DEBUG_BOUNDS device checks), loaded once
    beside libmla.so; the same C ABI."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


def _load(path):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "or python -m mla_latent_kv_05_amd.build")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    PP = ctypes.POINTER(Params)
    st = ctypes.c_int
    for name, args in (
        ("mla_absorb_q", [PP, P, P, P, P]),
        ("mla_decode_splitkv", [PP, P, P, P, P, P, P, P, P, P, P]),
        ("mla_combine_lse", [PP, P, P, P, P, P]),
        ("mla_up_v", [PP, P, P, P, P]),
        ("mla_combine_up_v", [PP, P, P, P, P, P, P]),
        ("mla_expand_kv", [PP, P, P, P, P]),
        ("mla_append_kv", [PP, P, P, P, P, P, P, P, P, P, P]),
        ("mla_decompress_kv", [PP, P, P, P, P, P, P, P, P]),
        ("mla_prefill_attention", [PP, P, P, P, P, P, P, P, P, P]),
        ("mla_decode_step", [PP, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int64, P]),
        ("mla_decode_step_noalloc", [PP, P, P, P, P, P, P, P, P, P, P, P, P]),
        ("mla_decode_step_persistent", [PP, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int64, P]),
        ("mla_check_params", [PP]),
        ("mla_plan_splits", [PP, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
    ):
        f = getattr(L, name)
        f.argtypes = args
        f.restype = st
    L.mla_decode_kernel_name.argtypes = [PP]
    L.mla_decode_kernel_name.restype = ctypes.c_char_p
    L.mla_status_string.argtypes = [st]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_last_error.argtypes = []
    L.mla_last_error.restype = ctypes.c_char_p
    L.mla_prefill_lmax.argtypes = [PP]
    L.mla_prefill_lmax.restype = ctypes.c_int64
    L.mla_prefer_absorbed.argtypes = [PP]
    L.mla_prefer_absorbed.restype = ctypes.c_int32
    L.mla_default_num_splits.argtypes = [PP, ctypes.c_int32]
    L.mla_default_num_splits.restype = ctypes.c_int32
    L.mla_decode_step_workspace.argtypes = [PP]
    L.mla_decode_step_workspace.restype = ctypes.c_int64
    L.mla_decode_step_persistent_workspace.argtypes = [PP]
    L.mla_decode_step_persistent_workspace.restype = ctypes.c_int64
    L.mla_abi_version.argtypes = []
    L.mla_abi_version.restype = ctypes.c_int32
    L.mla_device_errors.argtypes = [ctypes.POINTER(ctypes.c_uint32), P]
    L.mla_device_errors.restype = st
    L.mla_debug_bounds.argtypes = []
    L.mla_debug_bounds.restype = ctypes.c_int32
    if L.mla_abi_version() != 3:
        raise RuntimeError(f"{path}: ABI version mismatch")
    return L


def _check(status: int):
    if status != 0:
        raise MLAError(status, lib().mla_last_error().decode())


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    if t in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported dtype {t}")


def make_params(B: int, Sq: int, H: int, d_h: int, d_c: int, d_r: int, num_pages: int,
                max_pages: int, num_splits: int = 1, split_pages: Optional[int] = None,
                scale: Optional[float] = None, q_dtype: int = BF16, w_dtype: int = BF16,
                kv_dtype: int = BF16, pe_dtype: int = BF16, latent_dtype: int = BF16,
                out_dtype: int = F32, flags: int = 0, num_parts: int = 0, part_dtype: int = F32) -> Params:
    if split_pages is None:
        split_pages = -(-max_pages // num_splits)
    if scale is None:
        scale = 1.0 / math.sqrt(d_h + d_r)
    return Params(B, Sq, H, d_h, d_c, d_r, PAGE, num_pages, max_pages, num_splits, split_pages,
                  scale, q_dtype, w_dtype, kv_dtype, pe_dtype, latent_dtype, out_dtype, flags, num_parts, part_dtype)


def check_params(p: Params) -> None:
    _check(lib().mla_check_params(ctypes.byref(p)))


def plan_splits(p: Params, max_seq_len: int, total_tokens: int, num_cus: int = 256,
                min_splits: int = 1) -> Params:
    """Balanced split plan from the library's planner (host only): fills num_parts
    and num_splits."""
    q = p.copy()
    _check(lib().mla_plan_splits(ctypes.byref(q), max_seq_len, total_tokens, num_cus, min_splits))
    return q


def decode_kernel_name(p: Params) -> str:
    return lib().mla_decode_kernel_name(ctypes.byref(p)).decode()


def _ptr(t: Optional[torch.Tensor], what: str, shape=None, dtype: Optional[int] = None):
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError(f"{what}: must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)} != {tuple(shape)}")
    if dtype is not None and dtype_code(t.dtype) != dtype:
        raise ValueError(f"{what}: dtype {t.dtype} does not match the parameters")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def absorb_q(p: Params, q_nope, W_UK, q_abs, stream=None) -> None:
    rows = (p.B, p.Sq, p.H)
    _check(lib().mla_absorb_q(ctypes.byref(p),
                              _ptr(q_nope, "q_nope", rows + (p.d_h,), p.q_dtype),
                              _ptr(W_UK, "W_UK", (p.H, p.d_h, p.d_c), p.w_dtype),
                              _ptr(q_abs, "q_abs", rows + (p.d_c,), p.latent_dtype),
                              _stream(stream)))


def decode_splitkv(p: Params, q_abs, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens,
                   o_part, lse_part, stream=None) -> None:
    rows = (p.B, p.Sq, p.H)
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    _check(lib().mla_decode_splitkv(
        ctypes.byref(p),
        _ptr(q_abs, "q_abs", rows + (p.d_c,), p.latent_dtype),
        _ptr(q_rope, "q_rope", rows + (p.d_r,), p.q_dtype),
        _ptr(c_kv, "c_kv", (p.num_pages, PAGE, p.d_c), p.kv_dtype),
        _ptr(k_pe, "k_pe", (p.num_pages, PAGE, p.d_r), p.pe_dtype),
        _ptr(kv_scale, "kv_scale", (p.num_pages, PAGE), F32),
        _ptr(block_table, "block_table", (p.B, p.max_pages)),
        _ptr(seq_lens, "seq_lens", (p.B,)),
        _ptr(o_part, "o_part", rows + (p.num_splits, p.d_c), p.part_dtype),
        _ptr(lse_part, "lse_part", rows + (p.num_splits,), F32),
        _stream(stream)))


def combine_lse(p: Params, o_part, lse_part, o_latent, lse_out=None, stream=None) -> None:
    rows = (p.B, p.Sq, p.H)
    _check(lib().mla_combine_lse(ctypes.byref(p),
                                 _ptr(o_part, "o_part", rows + (p.num_splits, p.d_c), p.part_dtype),
                                 _ptr(lse_part, "lse_part", rows + (p.num_splits,), F32),
                                 _ptr(o_latent, "o_latent", rows + (p.d_c,), p.latent_dtype),
                                 _ptr(lse_out, "lse_out", rows, F32),
                                 _stream(stream)))


def up_v(p: Params, o_latent, W_UV, out, stream=None) -> None:
    rows = (p.B, p.Sq, p.H)
    _check(lib().mla_up_v(ctypes.byref(p),
                          _ptr(o_latent, "o_latent", rows + (p.d_c,), p.latent_dtype),
                          _ptr(W_UV, "W_UV", (p.H, p.d_h, p.d_c), p.w_dtype),
                          _ptr(out, "out", rows + (p.d_h,), p.out_dtype),
                          _stream(stream)))


def expand_kv(p: Params, c_kv, kv_scale, c_out, stream=None) -> None:
    """bf16 copy of an e4m3 cache with each token's scale applied: c_out = bf16(code * scale)."""
    _check(lib().mla_expand_kv(
        ctypes.byref(p),
        _ptr(c_kv, "c_kv", (p.num_pages, PAGE, p.d_c), FP8_E4M3),
        _ptr(kv_scale, "kv_scale", (p.num_pages, PAGE), F32),
        _ptr(c_out, "c_out", (p.num_pages, PAGE, p.d_c), BF16),
        _stream(stream)))


def combine_up_v(p: Params, o_part, lse_part, W_UV, out, lse_out=None, stream=None) -> None:
    """combine_lse followed by up_v in one launch (merged latent rows stay on chip)."""
    rows = (p.B, p.Sq, p.H)
    _check(lib().mla_combine_up_v(
        ctypes.byref(p),
        _ptr(o_part, "o_part", rows + (p.num_splits, p.d_c), p.part_dtype),
        _ptr(lse_part, "lse_part", rows + (p.num_splits,), F32),
        _ptr(W_UV, "W_UV", (p.H, p.d_h, p.d_c), p.w_dtype),
        _ptr(out, "out", rows + (p.d_h,), p.out_dtype),
        _ptr(lse_out, "lse_out", rows, F32),
        _stream(stream)))


DEVERR = {1: "MLA_DEVERR_SPLITS", 2: "MLA_DEVERR_SYNC", 4: "MLA_DEVERR_PAGE", 8: "MLA_DEVERR_SEQLEN", 16: "MLA_DEVERR_SCALE"}


def device_errors(stream=None, L=None) -> int:
    """Synchronise the stream and return (and clear) the device error bits the
    attention kernels raised since the last call (0 = none)."""
    L = lib() if L is None else L
    bits = ctypes.c_uint32(0)
    st = L.mla_device_errors(ctypes.byref(bits), _stream(stream))
    if st != 0:
        raise MLAError(st, L.mla_last_error().decode())
    return int(bits.value)


def decode_step_workspace(p: Params) -> int:
    """Bytes of device workspace decode_step needs for p."""
    r = lib().mla_decode_step_workspace(ctypes.byref(p))
    if r < 0:
        raise MLAError(2, lib().mla_last_error().decode())
    return int(r)


def decode_step(p: Params, q_nope, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, W_UK, W_UV, out,
                lse_out=None, workspace=None, stream=None) -> None:
    """The whole decode step in one library call (absorb, attention, merge and
    up-projection), its intermediates in `workspace` (a uint8 GPU tensor of at
    least decode_step_workspace(p) bytes)."""
    rows = (p.B, p.Sq, p.H)
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if workspace is None or workspace.dtype != torch.uint8:
        raise ValueError("workspace: a uint8 GPU tensor is required")
    _check(lib().mla_decode_step(
        ctypes.byref(p),
        _ptr(q_nope, "q_nope", rows + (p.d_h,), p.q_dtype),
        _ptr(q_rope, "q_rope", rows + (p.d_r,), p.q_dtype),
        _ptr(c_kv, "c_kv", (p.num_pages, PAGE, p.d_c), p.kv_dtype),
        _ptr(k_pe, "k_pe", (p.num_pages, PAGE, p.d_r), p.pe_dtype),
        _ptr(kv_scale, "kv_scale", (p.num_pages, PAGE), F32),
        _ptr(block_table, "block_table", (p.B, p.max_pages)),
        _ptr(seq_lens, "seq_lens", (p.B,)),
        _ptr(W_UK, "W_UK", (p.H, p.d_h, p.d_c), p.w_dtype),
        _ptr(W_UV, "W_UV", (p.H, p.d_h, p.d_c), p.w_dtype),
        _ptr(out, "out", rows + (p.d_h,), p.out_dtype),
        _ptr(lse_out, "lse_out", rows, F32),
        _ptr(workspace, "workspace"),
        ctypes.c_int64(workspace.numel()),
        _stream(stream)))


def decode_step_noalloc(p: Params, q_nope, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, W_UK, W_UV, out,
                        lse_out=None, stream=None) -> None:
    """decode_step with its intermediates in the library's static scratch (no
    allocation; calls on one GPU must not overlap)."""
    rows = (p.B, p.Sq, p.H)
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    _check(lib().mla_decode_step_noalloc(
        ctypes.byref(p),
        _ptr(q_nope, "q_nope", rows + (p.d_h,), p.q_dtype),
        _ptr(q_rope, "q_rope", rows + (p.d_r,), p.q_dtype),
        _ptr(c_kv, "c_kv", (p.num_pages, PAGE, p.d_c), p.kv_dtype),
        _ptr(k_pe, "k_pe", (p.num_pages, PAGE, p.d_r), p.pe_dtype),
        _ptr(kv_scale, "kv_scale", (p.num_pages, PAGE), F32),
        _ptr(block_table, "block_table", (p.B, p.max_pages)),
        _ptr(seq_lens, "seq_lens", (p.B,)),
        _ptr(W_UK, "W_UK", (p.H, p.d_h, p.d_c), p.w_dtype),
        _ptr(W_UV, "W_UV", (p.H, p.d_h, p.d_c), p.w_dtype),
        _ptr(out, "out", rows + (p.d_h,), p.out_dtype),
        _ptr(lse_out, "lse_out", rows, F32),
        _stream(stream)))


def append_kv(p: Params, c_new, kpe_new, block_table, seq_lens, c_kv, k_pe, kv_scale=None,
              q_rope_in=None, q_rope_out=None, stream=None) -> None:
    """Write the new tokens' latent rows and rotated RoPE keys into the cache
    (and rotate q_rope_in into q_rope_out, which may be the same tensor)."""
    tok = (p.B, p.Sq)
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    _check(lib().mla_append_kv(
        ctypes.byref(p),
        _ptr(c_new, "c_new", tok + (p.d_c,), p.q_dtype),
        _ptr(kpe_new, "kpe_new", tok + (p.d_r,), p.q_dtype),
        _ptr(q_rope_in, "q_rope_in", tok + (p.H, p.d_r), p.q_dtype),
        _ptr(q_rope_out, "q_rope_out", tok + (p.H, p.d_r), p.q_dtype),
        _ptr(block_table, "block_table", (p.B, p.max_pages)),
        _ptr(seq_lens, "seq_lens", (p.B,)),
        _ptr(c_kv, "c_kv", (p.num_pages, PAGE, p.d_c), p.kv_dtype),
        _ptr(k_pe, "k_pe", (p.num_pages, PAGE, p.d_r), p.pe_dtype),
        _ptr(kv_scale, "kv_scale", (p.num_pages, PAGE), F32),
        _stream(stream)))


def prefer_absorbed(p: Params) -> bool:
    """The switch of "MLA Matrix Absorption" sec. 6: True when p.Sq new tokens per
    sequence are served by the absorbed path (the four decode calls), False when by
    decompress_kv + prefill_attention."""
    r = lib().mla_prefer_absorbed(ctypes.byref(p))
    if r < 0:
        raise MLAError(2, lib().mla_last_error().decode())
    return bool(r)


def default_num_splits(p: Params, max_seq_len: int) -> int:
    """Fixed-split count per sequence that fills an MI355X for B sequences of
    max_seq_len tokens (use with split_pages = ceil(ceil(max_seq_len / 64) / S))."""
    r = lib().mla_default_num_splits(ctypes.byref(p), int(max_seq_len))
    if r < 0:
        raise MLAError(2, lib().mla_last_error().decode())
    return int(r)


def lmax(p: Params) -> int:
    """Row stride (positions) of the decompressed keys and values: max_pages * 64
    rounded up to a multiple of 256."""
    r = lib().mla_prefill_lmax(ctypes.byref(p))
    if r < 0:
        raise MLAError(2, lib().mla_last_error().decode())
    return int(r)


def decompress_kv(p: Params, c_kv, block_table, seq_lens, W_UK, W_UV, k_nope, v_t, stream=None) -> None:
    """Per-head keys k_nope [B, Lmax, H, d_h] and transposed values v_t [B, H, d_h, Lmax]
    of every cached position (non-absorbed path)."""
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    L = lmax(p)
    _check(lib().mla_decompress_kv(
        ctypes.byref(p),
        _ptr(c_kv, "c_kv", (p.num_pages, PAGE, p.d_c), p.kv_dtype),
        _ptr(block_table, "block_table", (p.B, p.max_pages)),
        _ptr(seq_lens, "seq_lens", (p.B,)),
        _ptr(W_UK, "W_UK", (p.H, p.d_h, p.d_c), p.w_dtype),
        _ptr(W_UV, "W_UV", (p.H, p.d_h, p.d_c), p.w_dtype),
        _ptr(k_nope, "k_nope", (p.B, L, p.H, p.d_h), p.latent_dtype),
        _ptr(v_t, "v_t", (p.B, p.H, p.d_h, L), p.latent_dtype),
        _stream(stream)))


def prefill_attention(p: Params, q_nope, q_rope, k_nope, v_t, k_pe, block_table, seq_lens, out,
                      stream=None) -> None:
    """Causal attention of the p.Sq new tokens with the decompressed keys and values."""
    rows = (p.B, p.Sq, p.H)
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    L = lmax(p)
    _check(lib().mla_prefill_attention(
        ctypes.byref(p),
        _ptr(q_nope, "q_nope", rows + (p.d_h,), p.q_dtype),
        _ptr(q_rope, "q_rope", rows + (p.d_r,), p.q_dtype),
        _ptr(k_nope, "k_nope", (p.B, L, p.H, p.d_h), p.latent_dtype),
        _ptr(v_t, "v_t", (p.B, p.H, p.d_h, L), p.latent_dtype),
        _ptr(k_pe, "k_pe", (p.num_pages, PAGE, p.d_r), p.pe_dtype),
        _ptr(block_table, "block_table", (p.B, p.max_pages)),
        _ptr(seq_lens, "seq_lens", (p.B,)),
        _ptr(out, "out", rows + (p.d_h,), p.out_dtype),
        _stream(stream)))


class BoundCalls:
    """The four calls of a decode step with their arguments checked and marshalled
    once: each call afterwards is a bare ctypes call (the library still validates
    the parameters on every call).  The tensors must stay alive and in place."""

    def __init__(self, p: Params, q_nope, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens,
                 W_UK, W_UV, q_abs, o_part, lse_part, o_latent, lse, out, stream=None, fused=False,
                 expand=None):
        rows = (p.B, p.Sq, p.H)
        self.fused = fused
        # expand = (decode parameters with a bf16 cache, the bf16 workspace): the step
        # expands the e4m3 cache first and attends to the copy
        pd = p if expand is None else expand[0]
        if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
            raise ValueError("block_table and seq_lens must be int32")
        self.p = p
        pp = ctypes.byref(p)
        st = _stream(stream)
        L = lib()
        self._calls = (
            (L.mla_absorb_q, (pp, _ptr(q_nope, "q_nope", rows + (p.d_h,), p.q_dtype),
                              _ptr(W_UK, "W_UK", (p.H, p.d_h, p.d_c), p.w_dtype),
                              _ptr(q_abs, "q_abs", rows + (p.d_c,), p.latent_dtype), st)),
            (L.mla_decode_splitkv, (ctypes.byref(pd), _ptr(q_abs, "q_abs", rows + (p.d_c,), p.latent_dtype),
                                    _ptr(q_rope, "q_rope", rows + (p.d_r,), p.q_dtype),
                                    _ptr(c_kv if expand is None else expand[1], "c_kv",
                                         (p.num_pages, PAGE, p.d_c), pd.kv_dtype),
                                    _ptr(k_pe, "k_pe", (p.num_pages, PAGE, p.d_r), p.pe_dtype),
                                    _ptr(kv_scale if expand is None else None, "kv_scale", (p.num_pages, PAGE), F32),
                                    _ptr(block_table, "block_table", (p.B, p.max_pages)),
                                    _ptr(seq_lens, "seq_lens", (p.B,)),
                                    _ptr(o_part, "o_part", rows + (p.num_splits, p.d_c), p.part_dtype),
                                    _ptr(lse_part, "lse_part", rows + (p.num_splits,), F32), st)),
            (L.mla_combine_lse, (pp, _ptr(o_part, "o_part", rows + (p.num_splits, p.d_c), p.part_dtype),
                                 _ptr(lse_part, "lse_part", rows + (p.num_splits,), F32),
                                 _ptr(o_latent, "o_latent", rows + (p.d_c,), p.latent_dtype),
                                 _ptr(lse, "lse_out", rows, F32), st)),
            (L.mla_up_v, (pp, _ptr(o_latent, "o_latent", rows + (p.d_c,), p.latent_dtype),
                          _ptr(W_UV, "W_UV", (p.H, p.d_h, p.d_c), p.w_dtype),
                          _ptr(out, "out", rows + (p.d_h,), p.out_dtype), st)),
            (L.mla_combine_up_v, (pp, _ptr(o_part, "o_part", rows + (p.num_splits, p.d_c), p.part_dtype),
                                  _ptr(lse_part, "lse_part", rows + (p.num_splits,), F32),
                                  _ptr(W_UV, "W_UV", (p.H, p.d_h, p.d_c), p.w_dtype),
                                  _ptr(out, "out", rows + (p.d_h,), p.out_dtype),
                                  _ptr(lse, "lse_out", rows, F32), st)),
        )
        self._step = (self._calls[0], self._calls[1], self._calls[4]) if fused else self._calls[:4]
        if expand is not None:
            ex = (L.mla_expand_kv, (pp, _ptr(c_kv, "c_kv", (p.num_pages, PAGE, p.d_c), FP8_E4M3),
                                    _ptr(kv_scale, "kv_scale", (p.num_pages, PAGE), F32),
                                    _ptr(expand[1], "c_out", (p.num_pages, PAGE, p.d_c), BF16), st))
            self._calls = self._calls + (ex,)
            self._step = (ex,) + self._step

    def expand_kv(self):
        f, a = self._calls[5]
        _check(f(*a))

    def absorb_q(self):
        f, a = self._calls[0]
        _check(f(*a))

    def decode_splitkv(self):
        f, a = self._calls[1]
        _check(f(*a))

    def combine_lse(self):
        f, a = self._calls[2]
        _check(f(*a))

    def up_v(self):
        f, a = self._calls[3]
        _check(f(*a))

    def combine_up_v(self):
        f, a = self._calls[4]
        _check(f(*a))

    def __call__(self):
        for f, a in self._step:
            _check(f(*a))


_TORCH = {F32: torch.float32, BF16: torch.bfloat16}


class DecodeStep:
    """Owns the intermediates of one decode step (allocated once with torch) and
    runs the four library calls on the current stream (fused=True: absorb, decode
    and the fused merge + up-projection; o_latent is then not written)."""

    def __init__(self, p: Params, device="cuda", fused=False, expand=False):
        self.p = p
        self.fused = fused
        # expand (e4m3 cache only): each step first expands the cache to a bf16 copy
        # (mla_expand_kv) and attends to it with the bf16 kernel
        self.expand = bool(expand) and p.kv_dtype == FP8_E4M3
        if self.expand:
            self.p_dec = p.copy()
            self.p_dec.kv_dtype = BF16
            self.kv_bf16 = torch.empty((p.num_pages, PAGE, p.d_c), dtype=torch.bfloat16, device=device)
        rows = (p.B, p.Sq, p.H)
        self.q_abs = torch.empty(rows + (p.d_c,), dtype=_TORCH[p.latent_dtype], device=device)
        self.o_part = torch.empty(rows + (p.num_splits, p.d_c), dtype=_TORCH[p.part_dtype], device=device)
        self.lse_part = torch.empty(rows + (p.num_splits,), dtype=torch.float32, device=device)
        self.o_latent = torch.empty(rows + (p.d_c,), dtype=_TORCH[p.latent_dtype], device=device)
        self.lse = torch.empty(rows, dtype=torch.float32, device=device)
        self.out = torch.empty(rows + (p.d_h,), dtype=_TORCH[p.out_dtype], device=device)

    def bind(self, q_nope, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, W_UK, W_UV,
             stream=None) -> BoundCalls:
        """The four calls on these inputs, marshalled once (see BoundCalls)."""
        return BoundCalls(self.p, q_nope, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, W_UK, W_UV,
                          self.q_abs, self.o_part, self.lse_part, self.o_latent, self.lse, self.out, stream,
                          fused=self.fused, expand=(self.p_dec, self.kv_bf16) if self.expand else None)

    def __call__(self, q_nope, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens, W_UK, W_UV,
                 stream=None):
        p = self.p
        if self.expand:
            expand_kv(p, c_kv, kv_scale, self.kv_bf16, stream)
        absorb_q(p, q_nope, W_UK, self.q_abs, stream)
        if self.expand:
            decode_splitkv(self.p_dec, self.q_abs, q_rope, self.kv_bf16, k_pe, None, block_table, seq_lens,
                           self.o_part, self.lse_part, stream)
        else:
            decode_splitkv(p, self.q_abs, q_rope, c_kv, k_pe, kv_scale, block_table, seq_lens,
                           self.o_part, self.lse_part, stream)
        if self.fused:
            combine_up_v(p, self.o_part, self.lse_part, W_UV, self.out, self.lse, stream)
        else:
            combine_lse(p, self.o_part, self.lse_part, self.o_latent, self.lse, stream)
            up_v(p, self.o_latent, W_UV, self.out, stream)
        return self.out


def decode_step_persistent_workspace(p: Params) -> int:
    """Bytes of device workspace decode_step_persistent needs for p (raises for an
    unsupported p)."""
    r = lib().mla_decode_step_persistent_workspace(ctypes.byref(p))
    if r < 0:
        raise MLAError(6, "mla_decode_step_persistent does not support these parameters")
    return int(r)


def decode_step_persistent(p: Params, q_nope, q_rope, c_kv, k_pe, block_table, seq_lens, W_UK, W_UV, out,
                           lse_out=None, workspace=None, stream=None) -> None:
    """The decode step of a small batch in one launch.  `workspace`: a
    uint8 GPU tensor of at least decode_step_persistent_workspace(p) bytes whose
    first 256 bytes are zero before its first use (torch.zeros); each call leaves
    them zero."""
    rows = (p.B, p.Sq, p.H)
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if workspace is None or workspace.dtype != torch.uint8:
        raise ValueError("workspace: a uint8 GPU tensor is required")
    _check(lib().mla_decode_step_persistent(
        ctypes.byref(p),
        _ptr(q_nope, "q_nope", rows + (p.d_h,), p.q_dtype),
        _ptr(q_rope, "q_rope", rows + (p.d_r,), p.q_dtype),
        _ptr(c_kv, "c_kv", (p.num_pages, PAGE, p.d_c), p.kv_dtype),
        _ptr(k_pe, "k_pe", (p.num_pages, PAGE, p.d_r), p.pe_dtype),
        _ptr(block_table, "block_table", (p.B, p.max_pages)),
        _ptr(seq_lens, "seq_lens", (p.B,)),
        _ptr(W_UK, "W_UK", (p.H, p.d_h, p.d_c), p.w_dtype),
        _ptr(W_UV, "W_UV", (p.H, p.d_h, p.d_c), p.w_dtype),
        _ptr(out, "out", rows + (p.d_h,), p.out_dtype),
        _ptr(lse_out, "lse_out", rows, F32),
        _ptr(workspace, "workspace"),
        ctypes.c_int64(workspace.numel()),
        _stream(stream)))
