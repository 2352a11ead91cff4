"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Error metric: max |gpu - oracle| / RMS(oracle) over the compared outputs.
Bounds: 1e-4 with fp32 inputs, 2e-2 with bf16 inputs, 6e-2 with an fp8 cache.
Small cases compare every output; the full-size workloads run in the launch
configuration the bench uses and compare sampled rows the oracle computes
one by one.
"""
import math
import sys

import numpy as np
import pytest
import torch

from mla_latent_kv_05_amd import inputs as I
from mla_latent_kv_05_amd import mla
from oracle import oracle as O
from tests.helpers import (TOL, DeviceCase, assert_bf16_rounding, err_rms, err_rows, params_for, sample_rows,
                           split_page_ranges)

pytestmark = pytest.mark.gpu


def validate(case: I.Case):
    """Host-side check that the block table and lengths respect the ABI preconditions."""
    lens = case.seq_lens.to(torch.int64)
    assert int(lens.min()) >= 0 and int(lens.max()) <= case.max_pages * 64
    for b in range(case.wl.B):
        n = -(-int(lens[b]) // 64)
        if n == 0:
            continue
        ids = case.block_table[b, :n]
        assert int(ids.min()) >= 0 and int(ids.max()) < case.num_pages


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tol_of(wl):
    return TOL[wl.dtype]


# ------------------------------------------------------------------ one entry point at a time

@pytest.mark.parametrize("wl_name,R,flags", [
    ("v3_b1", 1, 0), ("v3_b64", 3, 0), ("v3_b64", 8, 0),        # at most 8 rows: one workgroup per head half
    ("v3_b64", 64, 0), ("v3_b64", 70, 0), ("v3_sq4_fp8", 9, 0),
    ("v3_b64", 70, mla.FLAG_GENERIC), ("tiny", 3, 0),
])
def test_absorb_q(wl_name, R, flags):
    wl = I.workload(wl_name, B=R, Sq=1)
    case = I.make_case(wl, seq_lens=[64] * wl.B)
    p = params_for(case, flags=flags)
    note(f"absorb_q {wl_name} R={R} flags={flags}")
    qa = torch.empty((wl.B, wl.Sq, wl.H, wl.d_c), dtype=torch.float32 if wl.dtype == "f32" else torch.bfloat16,
                     device="cuda")
    mla.absorb_q(p, case.q_nope.cuda(), case.W_UK.cuda(), qa)
    torch.cuda.synchronize()
    ref = O.absorb_q(O.dims_of(case), case.q_nope, case.W_UK)
    e = err_rms(qa.float().cpu().numpy(), ref)
    note(f"  err {e:.3e}")
    if wl.dtype == "f32":
        assert e <= 1e-5
    else:
        assert e <= TOL["bf16"]
        assert_bf16_rounding(qa.float().cpu().numpy(), ref)


def test_absorb_q_small_batch_fp32_latent():
    """At most 8 query rows with an fp32 q_abs: the fp32 sums themselves, against
    the oracle in fp64 (bf16 inputs, 128 products per element)."""
    wl = I.workload("v3_b64", B=5)
    case = I.make_case(wl, seq_lens=[64] * wl.B)
    p = params_for(case)
    p.latent_dtype = mla.F32
    note("absorb_q small batch, fp32 q_abs")
    qa = torch.empty((wl.B, 1, wl.H, wl.d_c), dtype=torch.float32, device="cuda")
    dc = DeviceCase(case)
    mla.absorb_q(p, dc.q_nope, dc.W_UK, qa)
    torch.cuda.synchronize()
    ref = O.absorb_q(O.dims_of(case), case.q_nope, case.W_UK)
    assert err_rms(qa.cpu().numpy(), ref) <= 1e-5


def run_decode(case, p, ref=None):
    """The kernel's partials for p and the oracle's (ref: those of an earlier call
    with the same plan, reused)."""
    dc = DeviceCase(case)
    q_abs = I.random_q_abs(case.wl, seed=123)
    S = p.num_splits
    rows = (case.wl.B, case.wl.Sq, case.wl.H)
    pdt = torch.bfloat16 if p.part_dtype == mla.BF16 else torch.float32
    o_part = torch.full(rows + (S, case.wl.d_c), float("nan"), dtype=pdt, device="cuda")
    lse_part = torch.full(rows + (S,), float("nan"), device="cuda")
    mla.decode_splitkv(p, q_abs.cuda(), dc.q_rope, dc.c_kv, dc.k_pe, dc.kv_scale, dc.block_table,
                       dc.seq_lens, o_part, lse_part)
    torch.cuda.synchronize()
    if ref is None:
        beg, end = split_page_ranges(case.seq_lens.numpy(), p)
        ref = O.decode_page_ranges(O.dims_of(case), q_abs, case.q_rope, case.c_kv, case.kv_scale,
                                   case.k_pe, case.block_table, case.seq_lens, beg, end)
    return o_part.float().cpu().numpy(), lse_part.cpu().numpy(), ref[0], ref[1]


def kernel_variants(wl, flags):
    """Flag sets to run: where both bf16 attention kernels take the workload, each of
    them forced (small test grids would otherwise always get the 64-row kernel)."""
    if flags == 0 and wl.dtype == "bf16" and (wl.Sq * wl.H) % 128 == 0:
        return [mla.FLAG_ROWS128, mla.FLAG_ROWS64]
    return [flags]


def check_partials(wl, o, l, ref_o, ref_l, key_gain=1.0, part_bf16=False):
    """lse bounds as for a whole step (see test_step_matches_oracle): 2e-3 for a bf16
    cache, 6e-3 for e4m3 (a second rounding of the key); key_gain is how much larger
    than the generator's the keys may be, which scales both roundings' errors.  With
    bf16 partials each element's own rounding (at most 2^-9 of its value; 2^-8
    allowed) is taken off before the bound on o_part, as for a bf16 output."""
    empty = ref_l == -np.inf
    assert not np.isnan(l).any(), "an lse_part slot was left unwritten"
    assert np.array_equal(l == -np.inf, empty), "empty splits differ"
    full = ~empty
    if full.any():
        lse_tol = {"f32": 1e-5, "fp8": 6e-3}.get(wl.dtype, 2e-3) * key_gain
        assert np.abs(l[full] - ref_l[full]).max() <= lse_tol
        if part_bf16:
            d = np.maximum(np.abs(o[full].astype(np.float64) - ref_o[full]) - 2.0 ** -8 * np.abs(ref_o[full]), 0.0)
            e = float(d.max()) / float(np.sqrt(np.mean(ref_o[full] ** 2)))
        else:
            e = err_rms(o[full], ref_o[full])
        note(f"  o_part err {e:.3e}")
        assert e <= tol_of(wl)


@pytest.mark.parametrize("wl_name,lens,split_pages,flags", [
    ("v3_b64", [1, 63, 64, 65, 200, 700], 1, 0),
    ("v3_b64", [1, 63, 64, 65, 200, 700], 3, 0),
    ("v3_b64", [1, 63, 64, 65, 200, 700], 100, 0),
    ("v3_b64", [130, 5, 1000], 2, mla.FLAG_GENERIC),
    ("v3_sq4_fp8", [1, 2, 3, 4, 5, 66, 67, 500], 2, 0),
    ("v3_sq4_fp8", [4, 129, 700], 100, 0),
    ("v3_b64", [3, 64, 190], 1, 0),
    ("tiny", [128], 1, 0),
    ("tiny", [5, 77], 1, 0),
])
def test_decode_splitkv(wl_name, lens, split_pages, flags):
    wl = I.workload(wl_name, B=len(lens))
    case = I.make_case(wl, seq_lens=lens)
    validate(case)
    ref = None
    for fl in kernel_variants(wl, flags):
        p = params_for(case, split_pages=split_pages, flags=fl)
        note(f"decode_splitkv {wl_name} lens={lens} sp={split_pages} S={p.num_splits} "
             f"kernel={mla.decode_kernel_name(p)}")
        o, l, *ref = run_decode(case, p, ref)
        check_partials(wl, o, l, *ref)


@pytest.mark.parametrize("over,lens,extra", [
    ({}, [1, 63, 64, 65, 200, 700], 0),
    ({}, [0, 130, 1], 2),              # an empty sequence and spare split slots: lse -inf
    ({"H": 32}, [77, 300], 0),
    ({"H": 96}, [64, 129], 0),
    ({}, [4096], 0),                   # the DeepSeek-V3 B = 1 length
])
def test_page_kernel(over, lens, extra):
    """Fixed splits of one page with bf16 partials: the page kernel (one workgroup per
    page and 32 heads) against the oracle's page partials; a split past a sequence's
    pages reads lse = -inf."""
    wl = I.workload("v3_b64", B=len(lens), **over)
    case = I.make_case(wl, seq_lens=lens)
    validate(case)
    p = params_for(case, split_pages=1, part_dtype=mla.BF16)
    p.num_splits += extra
    note(f"page kernel {over} lens={lens} S={p.num_splits} kernel={mla.decode_kernel_name(p)}")
    assert mla.decode_kernel_name(p) == "page_bf16"
    o, l, ref_o, ref_l = run_decode(case, p)
    check_partials(wl, o, l, ref_o, ref_l, part_bf16=True)


@pytest.mark.parametrize("wl_name,lens,num_parts,extra_slots,flags", [
    ("v3_b64", [1, 63, 64, 65, 200, 700], 1, 0, 0),          # one part: every sequence whole
    ("v3_b64", [1, 63, 64, 65, 200, 700], 3, 0, 0),
    ("v3_b64", [1, 63, 64, 65, 200, 700], 7, 2, 0),          # spare slots must read -inf
    ("v3_b64", [1, 63, 64, 65, 200, 700], 40, 0, 0),         # more parts than pages: empty parts
    ("v3_b64", [0, 130, 0, 64, 0], 3, 1, 0),                 # empty sequences
    ("v3_b64", [5000, 3, 2, 4100], 16, 0, 0),                # long sequences over many parts
    ("v3_b64", [1, 63, 64, 65, 200, 700], 5, 0, mla.FLAG_GENERIC),
    ("v3_sq4_fp8", [1, 2, 3, 4, 5, 66, 67, 500], 5, 0, 0),
    ("v3_sq4_fp8", [4, 129, 700, 0], 3, 1, 0),
    ("tiny", [5, 77, 128], 2, 0, 0),
])
def test_decode_balanced_splits(wl_name, lens, num_parts, extra_slots, flags):
    wl = I.workload(wl_name, B=len(lens))
    case = I.make_case(wl, seq_lens=lens)
    validate(case)
    ref = None
    for fl in kernel_variants(wl, flags):
        p = params_for(case, num_parts=num_parts, flags=fl)
        p.num_splits += extra_slots
        note(f"balanced {wl_name} lens={lens} P={num_parts} S={p.num_splits} kernel={mla.decode_kernel_name(p)}")
        o, l, *ref = run_decode(case, p, ref)
        check_partials(wl, o, l, *ref)


@pytest.mark.parametrize("wl_name,over,lens,num_parts,flags", [
    ("v3_b64", {}, [1, 63, 64, 65, 200, 700], 5, mla.FLAG_ROWS128),   # four-wave kernel, 128 rows
    ("v3_b64", {}, [1, 63, 64, 65, 200, 700], 5, mla.FLAG_ROWS64),    # eight-wave kernel, 64 rows
    ("v3_b64", {"H": 64}, [1, 63, 64, 65, 200, 700], 5, 0),           # eight-wave kernel, 64 heads
    ("v3_sq4_fp8", {}, [4, 129, 700, 0], 3, 0),                        # e4m3 cache
    ("v3_b64", {}, [130, 5, 1000], 2, mla.FLAG_GENERIC),              # fp32 VALU kernel
])
def test_decode_bf16_partials(wl_name, over, lens, num_parts, flags):
    """part_dtype = BF16: the partials are the fp32 partials (checked against the
    oracle) rounded to nearest even, bit for bit, with the same lse values.  (Rounded
    partials are not held to the max-error bound itself: a split of a few tokens
    has values ~10x the RMS of all partials, where bf16's half ulp alone is 2%.)"""
    wl = I.workload(wl_name, B=len(lens), **over)
    case = I.make_case(wl, seq_lens=lens)
    validate(case)
    p = params_for(case, num_parts=num_parts, flags=flags)
    note(f"bf16 partials {wl_name} {over} lens={lens} P={num_parts} kernel={mla.decode_kernel_name(p)}")
    o32, l32, ref_o, ref_l = run_decode(case, p)
    pb = p.copy()
    pb.part_dtype = mla.BF16
    o16, l16, _, _ = run_decode(case, pb)
    check_partials(wl, o32, l32, ref_o, ref_l)
    assert np.array_equal(l16, l32)
    full = ref_l != -np.inf
    want = torch.from_numpy(o32[full]).bfloat16().float().numpy()
    assert np.array_equal(o16[full], want)


@pytest.mark.parametrize("lens,split_pages,num_parts,part,scales", [
    ([1, 66, 700, 9000], 1000, 0, mla.F32, "pow2"),     # whole sequences: a 141-page segment
    ([1, 66, 700, 9000], 1000, 0, mla.F32, "pow2-flag"),
    ([4, 129, 700, 0], 2, 0, mla.F32, "any"),
    ([4, 129, 700, 0], 2, 0, mla.F32, "pow2-flag"),
    ([5000, 3, 2, 4100], None, 16, mla.BF16, "pow2-flag"),   # balanced parts, bf16 partials
    ([5000, 3, 2, 4100], None, 16, mla.BF16, "any"),
    ([33, 64, 95, 10], 1, 0, mla.BF16, "pow2-flag"),         # ragged last tiles, one page per split
])
def test_e4m3_partials_equal_those_of_the_expanded_cache(lens, split_pages, num_parts, part, scales):
    """The kernel that reads the e4m3 cache converts each code as mla_expand_kv does
    (bf16 of the code times its token's scale): its partials equal, bit for bit,
    those of the bf16 kernel on the expanded cache, and match the oracle.  Scales:
    the generator's powers of two read the general way ("pow2") or with
    MLA_FLAG_POW2_SCALE's one-instruction conversion ("pow2-flag"), or scales that
    are no powers of two ("any": each multiplied by a factor in [1, 2))."""
    wl = I.workload("v3_sq4_fp8", B=len(lens))
    case = I.make_case(wl, seq_lens=lens)
    if scales == "any":
        f = torch.from_numpy(np.random.default_rng(9).uniform(1.0, 2.0, case.kv_scale.shape).astype(np.float32))
        case.kv_scale = (case.kv_scale * f).contiguous()
    validate(case)
    p = params_for(case, split_pages=split_pages, num_parts=num_parts, part_dtype=part,
                   flags=mla.FLAG_POW2_SCALE if scales == "pow2-flag" else 0)
    note(f"e4m3 vs expanded lens={lens} sp={split_pages} P={num_parts} S={p.num_splits} "
         f"kernel={mla.decode_kernel_name(p)}")
    dc = DeviceCase(case)
    q_abs = I.random_q_abs(wl, seed=123).cuda()
    rows = (wl.B, wl.Sq, wl.H)
    pdt = torch.bfloat16 if part == mla.BF16 else torch.float32
    res = []
    kv16 = torch.empty((case.num_pages, 64, wl.d_c), dtype=torch.bfloat16, device="cuda")
    mla.expand_kv(p, dc.c_kv, dc.kv_scale, kv16)
    pb = p.copy()
    pb.kv_dtype = mla.BF16
    pb.flags = mla.FLAG_ROWS128                   # the same kernel (small grids default to 64 rows)
    for pp, ckv, scl in ((p, dc.c_kv, dc.kv_scale), (pb, kv16, None)):
        o_part = torch.zeros(rows + (p.num_splits, wl.d_c), dtype=pdt, device="cuda")
        lse_part = torch.full(rows + (p.num_splits,), float("nan"), device="cuda")
        mla.decode_splitkv(pp, q_abs, dc.q_rope, ckv, dc.k_pe, scl, dc.block_table, dc.seq_lens, o_part, lse_part)
        res.append((o_part.float().cpu(), lse_part.cpu()))
    torch.cuda.synchronize()
    (o8, l8), (o16, l16) = res
    assert torch.equal(l8, l16)
    assert torch.equal(o8, o16)
    if part == mla.F32 and max(lens) <= 1000:
        beg, end = split_page_ranges(case.seq_lens.numpy(), p)
        ref_o, ref_l = O.decode_page_ranges(O.dims_of(case), q_abs.cpu(), case.q_rope, case.c_kv, case.kv_scale,
                                            case.k_pe, case.block_table, case.seq_lens, beg, end)
        check_partials(wl, o8.numpy(), l8.numpy(), ref_o, ref_l, key_gain=2.0 if scales == "any" else 1.0)


@pytest.mark.parametrize("wl_name,S,part", [("v3_b64", 7, mla.F32), ("tiny", 3, mla.F32), ("v3_sq4_fp8", 40, mla.F32),
                                             ("v3_b64", 7, mla.BF16), ("tiny", 3, mla.BF16), ("v3_b64", 70, mla.BF16)])
def test_combine_lse(wl_name, S, part):
    wl = I.workload(wl_name, B=3)
    o, l = I.random_partials(wl, S, seed=9)
    if part == mla.BF16:
        o = o.bfloat16()
    D = O.dims(wl.B, wl.Sq, wl.H, wl.d_h, wl.d_c, wl.d_r, S, wl.scale)
    ref_o, ref_l = O.combine_lse(D, o, l)
    latent = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    p = mla.make_params(wl.B, wl.Sq, wl.H, wl.d_h, wl.d_c, wl.d_r, 1, S, num_splits=S,
                        split_pages=1, latent_dtype=mla.dtype_code(latent), part_dtype=part)
    ol = torch.empty((wl.B, wl.Sq, wl.H, wl.d_c), dtype=latent, device="cuda")
    lse = torch.empty((wl.B, wl.Sq, wl.H), device="cuda")
    note(f"combine {wl_name} S={S} part={part}")
    mla.combine_lse(p, o.cuda(), l.cuda(), ol, lse)
    torch.cuda.synchronize()
    e = err_rms(ol.float().cpu().numpy(), ref_o)
    if wl.dtype == "f32":
        assert e <= 1e-5
    else:
        assert e <= TOL["bf16"]
        assert_bf16_rounding(ol.float().cpu().numpy(), ref_o)
    assert np.abs(lse.cpu().numpy() - ref_l).max() <= 1e-4


@pytest.mark.parametrize("wl_name,R,out_dtype,flags", [
    ("v3_b64", 64, mla.F32, 0), ("v3_b64", 70, mla.BF16, 0), ("v3_b1", 1, mla.F32, 0),
    ("v3_b64", 5, mla.F32, mla.FLAG_GENERIC), ("tiny", 4, mla.F32, 0),
])
def test_up_v(wl_name, R, out_dtype, flags):
    wl = I.workload(wl_name, B=R, Sq=1)
    case = I.make_case(wl, seq_lens=[64] * R)
    ol = I.random_o_latent(wl, seed=5)
    p = params_for(case, flags=flags, out_dtype=out_dtype)
    out = torch.empty((wl.B, 1, wl.H, wl.d_h), dtype=torch.float32 if out_dtype == mla.F32 else torch.bfloat16,
                      device="cuda")
    note(f"up_v {wl_name} R={R} out={out_dtype} flags={flags}")
    mla.up_v(p, ol.cuda(), case.W_UV.cuda(), out)
    torch.cuda.synchronize()
    ref = O.up_v(O.dims_of(case), ol, case.W_UV)
    e = err_rms(out.float().cpu().numpy(), ref)
    note(f"  err {e:.3e}")
    if wl.dtype == "f32" or out_dtype == mla.F32:
        assert e <= 1e-4
    else:
        assert e <= TOL["bf16"]
        assert_bf16_rounding(out.float().cpu().numpy(), ref)


# ------------------------------------------------------------------ the whole step, every output

SMALL = [
    ("tiny", {}, None),                                        # full size: B=1, L=128, fp32
    ("v3_b1", {}, None),                                       # full size: B=1, L=4096
    ("v3_b64", {"B": 6}, None),
    ("v3_long", {"B": 2, "seq_lo": 8192, "seq_hi": 8192}, None),
    ("v3_sq4_fp8", {"B": 4, "seq_lo": 300, "seq_hi": 2000}, None),
    ("v3_sq4_fp8", {"B": 3}, [4, 3, 66]),
    ("v3_b64", {"B": 3, "Sq": 32}, [40, 300, 1000]),          # many new tokens on the absorbed path
    ("v3_b64", {"B": 2, "Sq": 64}, [64, 700]),                # whole prompt of 64 tokens; a prefix
    ("v3_sq4_fp8", {"B": 2, "Sq": 32}, [40, 900]),            # the same on the e4m3 cache
]


@pytest.mark.parametrize("wl_name,over,lens", SMALL)
def test_step_matches_oracle(wl_name, over, lens):
    wl = I.workload(wl_name, **over)
    case = I.make_case(wl, seq_lens=lens)
    validate(case)
    p = params_for(case, plan=True)
    note(f"step {wl_name} {over} lens={case.seq_lens.tolist()[:8]} S={p.num_splits} sp={p.split_pages}")
    st = DeviceCase(case).step(p)
    torch.cuda.synchronize()
    out, ol, lse = O.decode(case)
    # many new tokens per sequence: rows see from a few positions to thousands, so
    # the error is taken per row (a few-position row returns values at full size)
    e = (err_rows if wl.Sq >= 16 else err_rms)(st.out.float().cpu().numpy(), out)
    note(f"  out err {e:.3e}")
    assert e <= tol_of(wl)
    vis = lse > -np.inf
    # lse: a row that sees one position returns that one score, whose error from the
    # bf16 absorbed query is about scale * 2^-9 * |q_abs| / sqrt(3) ~ 4e-4 (one sigma)
    # at these distributions; with many new tokens such rows exist, so 4e-3 (10 sigma).
    # e4m3: the cache enters the product as bf16(code x scale), a second rounding of
    # the same size (one score: about 6e-4 from either rounding, 9e-4 from both), so
    # 6e-3 (7 sigma).
    if wl.dtype == "f32":
        lse_tol = 1e-5
    elif wl.dtype == "fp8":
        lse_tol = 6e-3
    else:
        lse_tol = 4e-3 if wl.Sq >= 16 else 2e-3
    assert np.abs(st.lse.cpu().numpy()[vis] - lse[vis]).max() <= lse_tol
    assert np.all(st.lse.cpu().numpy()[~vis] == -np.inf)


def test_generic_path_matches_oracle_at_v3_shapes():
    wl = I.workload("v3_b64", B=3, Sq=2)
    case = I.make_case(wl, seq_lens=[70, 2, 300])
    p = params_for(case, split_pages=2, flags=mla.FLAG_GENERIC)
    st = DeviceCase(case).step(p)
    torch.cuda.synchronize()
    out, _, _ = O.decode(case)
    assert err_rms(st.out.float().cpu().numpy(), out) <= TOL["bf16"]


# ------------------------------------------------------------------ invariances and edge cases

def test_split_count_invariance():
    wl = I.workload("v3_b64", B=2, seq_lo=4096, seq_hi=4096)
    case = I.make_case(wl)
    dc = DeviceCase(case)
    outs = []
    for S in (1, 2, 8, 32, 64):
        p = params_for(case, num_splits=S)
        note(f"split invariance S={S} sp={p.split_pages}")
        outs.append(dc.step(p).out.cpu().numpy())
    torch.cuda.synchronize()
    ref, _, _ = O.decode(case)
    for o in outs:
        assert err_rms(o, ref) <= TOL["bf16"]
    for o in outs[1:]:
        assert err_rms(o, outs[0]) <= TOL["bf16"]


def test_physical_page_order_and_padding_contents_do_not_matter():
    """Permuting physical pages (with the block table) gives bitwise-identical output,
    and NaN in the unused slots of last pages changes nothing."""
    for name in ("v3_b64", "v3_sq4_fp8"):
        wl = I.workload(name, B=3)
        case = I.make_case(wl, seq_lens=[100, 4, 250])
        p = params_for(case, split_pages=2)
        a = DeviceCase(case).step(p).out.cpu()
        perm = torch.randperm(case.num_pages, generator=torch.Generator().manual_seed(2))
        inv = torch.argsort(perm).int()
        case2 = I.Case(**{**case.__dict__})
        case2.c_kv = case.c_kv[perm].contiguous()
        case2.k_pe = case.k_pe[perm].contiguous()
        if case.kv_scale is not None:
            case2.kv_scale = case.kv_scale[perm].contiguous()
        case2.block_table = torch.where(case.block_table >= 0, inv[case.block_table.clamp(min=0)],
                                        case.block_table).contiguous()
        b = DeviceCase(case2).step(p).out.cpu()
        assert torch.equal(a, b), name
        # poison every slot past the end of each sequence
        case3 = I.Case(**{**case.__dict__})
        case3.c_kv = case.c_kv.clone()
        case3.k_pe = case.k_pe.clone()
        case3.kv_scale = None if case.kv_scale is None else case.kv_scale.clone()
        for bb, n in enumerate(case.seq_lens.tolist()):
            if n % 64:
                pg = int(case.block_table[bb, n // 64])
                if case.kv_scale is None:
                    case3.c_kv[pg, n % 64:] = float("nan")
                else:
                    case3.c_kv[pg, n % 64:] = 0x7F             # e4m3 NaN code
                    case3.kv_scale[pg, n % 64:] = float("nan")
                case3.k_pe[pg, n % 64:] = float("nan")
        c = DeviceCase(case3).step(p).out.cpu()
        assert torch.equal(a, c), name


def test_causal_row_equals_shorter_single_row_run():
    wl4 = I.workload("v3_sq4_fp8", B=2)
    case = I.make_case(wl4, seq_lens=[300, 70])
    p4 = params_for(case, split_pages=2)
    out4 = DeviceCase(case).step(p4).out.cpu().numpy()
    for s in range(4):
        wl1 = I.workload("v3_sq4_fp8", B=2, Sq=1)
        c1 = I.Case(**{**case.__dict__, "wl": wl1, "seq_lens": (case.seq_lens - 3 + s).contiguous(),
                       "q_nope": case.q_nope[:, s:s + 1].contiguous(),
                       "q_rope": case.q_rope[:, s:s + 1].contiguous()})
        p1 = params_for(c1, split_pages=2)
        out1 = DeviceCase(c1).step(p1).out.cpu().numpy()
        assert err_rms(out4[:, s], out1[:, 0]) <= 1e-3


def test_degenerate_lengths():
    """seq_len < Sq leaves leading query rows with nothing visible: zero output, lse -inf."""
    wl = I.workload("v3_sq4_fp8", B=3)
    case = I.make_case(wl, seq_lens=[1, 2, 64])
    p = params_for(case, split_pages=1)
    st = DeviceCase(case).step(p)
    torch.cuda.synchronize()
    out, _, lse = O.decode(case)
    got_l = st.lse.cpu().numpy()
    assert np.array_equal(got_l == -np.inf, lse == -np.inf)
    assert np.all(st.out.cpu().numpy()[lse == -np.inf] == 0)
    assert err_rms(st.out.cpu().numpy(), out) <= TOL["fp8"]


def rising_case(name, factor=64.0):
    """Two sequences whose tokens past the first page have their latent and RoPE
    rows scaled by `factor` (e4m3: the token scales), so that the scores of a split
    starting at page 0 rise far above the maximum of its first tile, and those of
    later splits rise by varying amounts.  e4m3: the token scales are rounded to
    powers of two first, so that code x scale is exact in bf16 (scores of a few
    hundred would otherwise turn the cache's bf16 rounding into large weight errors)."""
    wl = I.workload(name, B=2)
    case = I.make_case(wl, seq_lens=[700, 300])
    if case.kv_scale is not None:
        case.kv_scale = torch.exp2(torch.round(torch.log2(case.kv_scale)))
    pages = set()
    for b, n in enumerate(case.seq_lens.tolist()):
        pages.update(int(x) for x in case.block_table[b, 1:-(-n // 64)].tolist())
    idx = torch.tensor(sorted(pages), dtype=torch.int64)
    if case.kv_scale is not None:
        case.kv_scale[idx] *= factor
    else:
        case.c_kv[idx] = (case.c_kv[idx].float() * factor).to(case.c_kv.dtype)
    case.k_pe[idx] = (case.k_pe[idx].float() * factor).to(case.k_pe.dtype)
    return case


def first_tile_excess(case, q_abs, b, n_split_tokens):
    """Per query row of sequence b: the largest score (log2 units) among its first
    n_split_tokens tokens minus the largest among the first 32."""
    qa = O.decode_values(q_abs)[b]
    qr = O.decode_values(case.q_rope)[b]
    n = int(case.seq_lens[b])
    pages = case.block_table[b, :-(-n // 64)].tolist()
    c = np.concatenate([O.cache_values(case)[pg] for pg in pages])[:n_split_tokens]
    k = np.concatenate([O.decode_values(case.k_pe)[pg] for pg in pages])[:n_split_tokens]
    z = (np.einsum("shc,tc->sht", qa, c) + np.einsum("shr,tr->sht", qr, k)) * case.wl.scale / math.log(2)
    return z.max(-1) - z[..., :32].max(-1)


@pytest.mark.parametrize("name", ["v3_b64", "v3_sq4_fp8"])
def test_second_pass_when_scores_rise_along_a_split(name):
    """Scores that rise along a split by more than 2^64 over the maximum of its first
    tile make the bf16 and e4m3 kernels compute the split again with the split's own
    maximum as the reference: the partials stay finite and match the oracle (run on
    the same bf16 q_abs, so that scores of a few hundred do not magnify its rounding)."""
    case = rising_case(name)
    q_abs = I.random_q_abs(case.wl, seed=123)              # the q_abs run_decode passes
    assert first_tile_excess(case, q_abs, 0, 256).min() > 64   # every row of split 0 of sequence 0
    for split_pages in (4, 16):
        ref = None
        for fl in kernel_variants(case.wl, 0):
            p = params_for(case, split_pages=split_pages, flags=fl)
            note(f"{name} rising scores split_pages={split_pages} kernel={mla.decode_kernel_name(p)}")
            o, l, *ref = run_decode(case, p, ref)
            assert np.isfinite(o[ref[1] != -np.inf]).all() and not np.isnan(l).any()
            check_partials(case.wl, o, l, *ref)


def test_wide_block_table_and_unreferenced_pages():
    wl = I.workload("v3_b64", B=2)
    case = I.make_case(wl, seq_lens=[65, 130], max_pages=40, extra_pages=5)
    validate(case)
    p = params_for(case, split_pages=3)
    st = DeviceCase(case).step(p)
    torch.cuda.synchronize()
    out, _, _ = O.decode(case)
    assert err_rms(st.out.cpu().numpy(), out) <= TOL["bf16"]


def test_repeatable_bitwise():
    wl = I.workload("v3_b64", B=4)
    case = I.make_case(wl)
    p = params_for(case, plan=True)
    dc = DeviceCase(case)
    a = dc.step(p).out.cpu()
    b = dc.step(p).out.cpu()
    assert torch.equal(a, b)


# ------------------------------------------------------------------ full-size workloads, sampled rows

FULL = [
    ("v3_b64", 6, 24, False),       # B=64, L ~ U[1024, 8192], permuted pages
    ("v3_long", 2, 12, False),      # B=4, L = 131072, >= 32 splits
    ("v3_sq4_fp8", 4, 12, False),   # B=128, Sq=4, L ~ U[4096, 16384], e4m3 cache
    ("v3_sq4_fp8", 4, 12, True),    # ... through the bf16 expansion of the cache
]


def bench_step(case, expand=False):
    """The step in the launch configuration the bench times: balanced plan, bf16
    partials (bf16 and e4m3 caches), the fused tail, the power-of-two scale flag for
    an e4m3 cache (the generator writes such scales, as the append does)."""
    wl = case.wl
    p = params_for(case, plan=True, part_dtype=mla.F32 if wl.dtype == "f32" else mla.BF16,
                   flags=mla.FLAG_POW2_SCALE if wl.dtype == "fp8" else 0)
    dc = DeviceCase(case)
    st = mla.DecodeStep(p, fused=True, expand=expand)
    st(dc.q_nope, dc.q_rope, dc.c_kv, dc.k_pe, dc.kv_scale, dc.block_table, dc.seq_lens, dc.W_UK, dc.W_UV)
    torch.cuda.synchronize()
    return p, st


@pytest.mark.parametrize("wl_name,n_seq,n_heads,expand", FULL)
def test_full_size_sampled(wl_name, n_seq, n_heads, expand):
    wl = I.workload(wl_name)
    note(f"full {wl_name} expand={expand}: generating")
    case = I.make_case(wl)
    validate(case)
    p, st = bench_step(case, expand)
    note(f"full {wl_name}: tokens={case.total_tokens} pages={case.num_pages} P={p.num_parts} S={p.num_splits} "
         f"kernel={mla.decode_kernel_name(p)}")
    got = st.out.float().cpu().numpy().reshape(-1, wl.d_h)
    got_l = st.lse.cpu().numpy().reshape(-1)
    assert np.isfinite(got).all()
    rows = sample_rows(case, n_seq, n_heads)
    note(f"full {wl_name}: oracle on {len(rows)} rows")
    out, _, lse = O.decode(case, rows=rows)
    e = err_rms(got[rows], out)
    note(f"  sampled out err {e:.3e}")
    assert e <= tol_of(wl)
    assert np.abs(got_l[rows] - lse).max() <= 2e-3


def test_full_size_every_row_b64():
    """Every output row of the B = 64 workload (8,192 rows, L ~ U[1024, 8192]) in
    the bench's launch configuration against the oracle."""
    wl = I.workload("v3_b64")
    case = I.make_case(wl)
    validate(case)
    p, st = bench_step(case)
    got = st.out.float().cpu().numpy().reshape(-1, wl.d_h)
    got_l = st.lse.cpu().numpy().reshape(-1)
    note(f"every row v3_b64: oracle on {got.shape[0]} rows")
    out, _, lse = O.decode(case)
    out = out.reshape(-1, wl.d_h)
    e = err_rms(got, out)
    rows_e = err_rows(got, out)
    note(f"  out err {e:.3e}, worst row {rows_e:.3e}")
    assert e <= tol_of(wl)
    assert np.abs(got_l - lse.reshape(-1)).max() <= 2e-3


def test_bound_calls_match_unbound():
    """The pre-marshalled calls the bench uses give bit-identical results to the
    per-call binding (same kernels, same arguments)."""
    wl = I.workload("v3_b64", B=5)
    case = I.make_case(wl, seq_lens=[1, 64, 700, 3000, 5000])
    validate(case)
    p = params_for(case, plan=True)
    dc = DeviceCase(case)
    note("bound calls vs per-call binding")
    st = dc.step(p)
    torch.cuda.synchronize()
    ref = st.out.clone()
    st.out.zero_()
    b = st.bind(dc.q_nope, dc.q_rope, dc.c_kv, dc.k_pe, dc.kv_scale, dc.block_table, dc.seq_lens, dc.W_UK, dc.W_UV)
    b()
    b()
    torch.cuda.synchronize()
    assert torch.equal(st.out, ref)
