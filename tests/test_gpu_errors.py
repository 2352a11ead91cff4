"""The device error word (mla_device_errors) through the C ABI: a stale split plan
is flagged, and the MLA_DEBUG_BOUNDS build (libmla_debug.so) flags out-of-range
block-table entries and lengths, replacing them with in-range values so that no
kernel reads outside its buffers.  Invalid inputs are only ever given to the
debug build."""
import ctypes
import sys

import pytest
import torch

from mla_latent_kv_05_amd import inputs as I
from mla_latent_kv_05_amd import mla
from tests.helpers import DeviceCase, params_for

pytestmark = pytest.mark.gpu

SPLITS, SYNC, PAGE, SEQLEN, SCALE = 1, 2, 4, 8, 16


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def decode(L, p, dc, q_abs, block_table=None, seq_lens=None):
    rows = (p.B, p.Sq, p.H)
    o = torch.zeros(rows + (p.num_splits, p.d_c), device="cuda")
    lse = torch.zeros(rows + (p.num_splits,), device="cuda")
    bt = dc.block_table if block_table is None else block_table
    sl = dc.seq_lens if seq_lens is None else seq_lens
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.mla_decode_splitkv(ctypes.byref(p), ptr(q_abs), ptr(dc.q_rope), ptr(dc.c_kv), ptr(dc.k_pe),
                                ptr(dc.kv_scale), ptr(bt), ptr(sl), ptr(o), ptr(lse), st) == 0, \
        L.mla_last_error().decode()
    return o, lse, mla.device_errors(L=L)


CASES = [("v3_b64", {}, mla.FLAG_ROWS128), ("v3_b64", {}, mla.FLAG_ROWS64), ("v3_b64", {"H": 64}, 0),
         ("v3_sq4_fp8", {}, 0), ("v3_b64", {}, mla.FLAG_GENERIC), ("v3_sq4_fp8", {}, mla.FLAG_POW2_SCALE)]


@pytest.mark.parametrize("wl_name,over,flags", CASES)
def test_stale_plan_is_flagged(wl_name, over, flags):
    """num_splits below the parts a sequence touches: the pages of the missing
    slots are skipped (never written out of range) and MLA_DEVERR_SPLITS is set."""
    lens = [5000, 3, 2, 4100]
    wl = I.workload(wl_name, B=len(lens), **over)
    case = I.make_case(wl, seq_lens=lens)
    dc = DeviceCase(case)
    q_abs = I.random_q_abs(wl, seed=5).cuda()
    p = params_for(case, num_parts=16, flags=flags)
    L = mla.lib()
    mla.device_errors(L=L)                                    # start clean
    note(f"stale plan {wl_name} {over} kernel={mla.decode_kernel_name(p)} S={p.num_splits}")
    assert decode(L, p, dc, q_abs)[2] == 0                    # the plan's bound: no error
    p.num_splits = 2                                          # the long sequences touch more parts
    assert decode(L, p, dc, q_abs)[2] == SPLITS


@pytest.mark.parametrize("wl_name,over,flags", [CASES[0], CASES[2], CASES[3], CASES[5]])
def test_debug_build_flags_bad_pages_and_lengths(wl_name, over, flags):
    D = mla.debug_lib()
    assert D.mla_debug_bounds() == 1 and mla.lib().mla_debug_bounds() == 0
    lens = [700, 130, 64]
    wl = I.workload(wl_name, B=len(lens), **over)
    case = I.make_case(wl, seq_lens=lens)
    dc = DeviceCase(case)
    q_abs = I.random_q_abs(wl, seed=6).cuda()
    p = params_for(case, num_parts=5, flags=flags)
    mla.device_errors(L=D)
    note(f"debug build {wl_name} kernel={mla.decode_kernel_name(p)}")
    # valid inputs: no error, and the same partials as the release build
    o_d, l_d, err = decode(D, p, dc, q_abs)
    assert err == 0
    o_r, l_r, err = decode(mla.lib(), p, dc, q_abs)
    assert err == 0
    assert torch.equal(o_d, o_r) and torch.equal(l_d, l_r)
    # a page past the cache and a negative one
    for bad in (case.num_pages + 1000, -5):
        bt = dc.block_table.clone()
        bt[0, 3] = bad
        assert decode(D, p, dc, q_abs, block_table=bt)[2] == PAGE, bad
    # a length past the block table's row
    sl = dc.seq_lens.clone()
    sl[1] = p.max_pages * 64 + 100
    assert decode(D, p, dc, q_abs, seq_lens=sl)[2] & SEQLEN


def test_debug_build_flags_a_scale_that_is_no_power_of_two():
    """MLA_FLAG_POW2_SCALE states that the e4m3 scales are powers of two; the debug
    build checks it for every row it converts (a scale past a sequence's end is not
    counted) and raises MLA_DEVERR_SCALE, and without the flag the same cache is
    read exactly (the bf16 kernel on its expansion gives the same partials)."""
    D = mla.debug_lib()
    lens = [700, 130, 64]
    wl = I.workload("v3_sq4_fp8", B=len(lens))
    case = I.make_case(wl, seq_lens=lens)
    for b, n in enumerate(lens):                   # the generator's scales, on valid rows
        t = torch.arange(n)
        rows = case.kv_scale[case.block_table[b, t // 64].long(), t % 64]
        assert bool(((rows.view(torch.int32) & 0x7fffff) == 0).all())
    dc = DeviceCase(case)
    q_abs = I.random_q_abs(wl, seed=7).cuda()
    p = params_for(case, num_parts=5, flags=mla.FLAG_POW2_SCALE)
    mla.device_errors(L=D)
    assert decode(D, p, dc, q_abs)[2] == 0
    # one valid row with a scale of 1.5 x a power of two: flagged with the flag
    pg = int(case.block_table[1, 0])
    dc.kv_scale[pg, 5] *= 1.5
    assert decode(D, p, dc, q_abs)[2] == SCALE
    # without the flag the row is read exactly, as on the expanded cache
    q = p.copy()
    q.flags = 0
    o8, l8, err = decode(mla.lib(), q, dc, q_abs)
    assert err == 0
    kv16 = torch.empty((case.num_pages, 64, wl.d_c), dtype=torch.bfloat16, device="cuda")
    mla.expand_kv(q, dc.c_kv, dc.kv_scale, kv16)
    qb = q.copy()
    qb.kv_dtype = mla.BF16
    qb.flags = mla.FLAG_ROWS128
    dc16 = DeviceCase(case)
    dc16.c_kv = kv16
    dc16.kv_scale = None
    o16, l16, err = decode(mla.lib(), qb, dc16, q_abs)
    assert err == 0
    assert torch.equal(o8, o16) and torch.equal(l8, l16)


def test_page_kernel_errors():
    """The page kernel (fixed one-page splits, bf16 partials): too few splits for the
    block table are refused on the host (MLA_ERR_SPLITS, nothing launched), and the
    debug build flags an out-of-range page and length and matches the release build
    on valid input."""
    lens = [700, 3]
    wl = I.workload("v3_b64", B=len(lens))
    case = I.make_case(wl, seq_lens=lens)
    dc = DeviceCase(case)
    q_abs = I.random_q_abs(wl, seed=8).cuda()
    p = params_for(case, split_pages=1, part_dtype=mla.BF16)
    note(f"page kernel errors kernel={mla.decode_kernel_name(p)} S={p.num_splits}")
    assert mla.decode_kernel_name(p) == "page_bf16"
    L, D = mla.lib(), mla.debug_lib()
    mla.device_errors(L=L)
    mla.device_errors(L=D)
    o_r, l_r, err = decode(L, p, dc, q_abs)
    assert err == 0
    o_d, l_d, err = decode(D, p, dc, q_abs)
    assert err == 0
    assert torch.equal(o_d, o_r) and torch.equal(l_d, l_r)
    q = p.copy()
    q.num_splits = 2                                         # 700 positions need 11 one-page splits
    o = torch.zeros((wl.B, 1, wl.H, 2, wl.d_c), device="cuda")
    lse = torch.zeros((wl.B, 1, wl.H, 2), device="cuda")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.mla_decode_splitkv(ctypes.byref(q), ptr(q_abs), ptr(dc.q_rope), ptr(dc.c_kv), ptr(dc.k_pe), None,
                                ptr(dc.block_table), ptr(dc.seq_lens), ptr(o), ptr(lse), st) == 4   # MLA_ERR_SPLITS
    bt = dc.block_table.clone()
    bt[0, 3] = case.num_pages + 1000
    assert decode(D, p, dc, q_abs, block_table=bt)[2] == PAGE
    sl = dc.seq_lens.clone()
    sl[1] = p.max_pages * 64 + 100
    assert decode(D, p, dc, q_abs, seq_lens=sl)[2] & SEQLEN
