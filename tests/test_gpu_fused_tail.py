"""The fused decode tail (mla_combine_up_v) through the C ABI: bit for bit the
result of mla_combine_lse followed by mla_up_v with a bf16 latent, and within
the bf16 tolerance of the oracle's merge and up-projection.  The whole step with
the fused tail equals the four-call step bit for bit."""
import sys

import numpy as np
import pytest
import torch

from mla_latent_kv_05_amd import inputs as I
from mla_latent_kv_05_amd import mla
from oracle import oracle as O
from tests.helpers import TOL, DeviceCase, err_rms, params_for

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("B,Sq,S,out_dtype,with_lse,part", [
    (64, 1, 3, mla.F32, True, mla.F32),       # two 32-row chunks per head
    (37, 4, 7, mla.BF16, True, mla.F32),      # 148 rows: a ragged last chunk
    (5, 1, 70, mla.F32, False, mla.F32),      # more splits than lanes
    (1, 1, 1, mla.F32, True, mla.F32),        # one row, one split
    (64, 1, 3, mla.F32, True, mla.BF16),      # bf16 partials
    (37, 4, 70, mla.F32, True, mla.BF16),
    # at most 8 rows per head: the whole workgroup merges one row at a time
    (1, 1, 32, mla.F32, True, mla.BF16),      # one row, 32 splits (B = 1 decode)
    (8, 1, 64, mla.BF16, True, mla.BF16),     # 8 rows, 64 splits
    (2, 4, 130, mla.F32, True, mla.BF16),     # 8 rows, three groups of 64 splits
    (3, 1, 40, mla.F32, True, mla.F32),       # fp32 partials: 32 staged per round
])
def test_combine_up_v_equals_two_calls(B, Sq, S, out_dtype, with_lse, part):
    wl = I.workload("v3_b64", B=B, Sq=Sq)
    o, l = I.random_partials(wl, S, seed=11)
    if part == mla.BF16:
        o = o.bfloat16()
    W_UV = I.make_case(I.workload("v3_b64", B=1), seq_lens=[64]).W_UV
    p = mla.make_params(B, Sq, wl.H, wl.d_h, wl.d_c, wl.d_r, 1, S, num_splits=S, split_pages=1,
                        out_dtype=out_dtype, part_dtype=part)
    td = torch.float32 if out_dtype == mla.F32 else torch.bfloat16
    od, ld, wd = o.cuda(), l.cuda(), W_UV.cuda()
    ol = torch.empty((B, Sq, wl.H, wl.d_c), dtype=torch.bfloat16, device="cuda")
    out_ref = torch.empty((B, Sq, wl.H, wl.d_h), dtype=td, device="cuda")
    lse_ref = torch.empty((B, Sq, wl.H), device="cuda")
    out = torch.full_like(out_ref, 7.0)
    lse = torch.full_like(lse_ref, 7.0) if with_lse else None
    note(f"combine_up_v B={B} Sq={Sq} S={S} out={out_dtype} lse={with_lse} part={part}")
    mla.combine_lse(p, od, ld, ol, lse_ref)
    mla.up_v(p, ol, wd, out_ref)
    mla.combine_up_v(p, od, ld, wd, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    if with_lse:
        assert torch.equal(lse, lse_ref)
    # and against the oracle's merge followed by its up-projection
    D = O.dims(B, Sq, wl.H, wl.d_h, wl.d_c, wl.d_r, S, wl.scale)
    ref_o, _ = O.combine_lse(D, o, l)
    ref = O.up_v(D, torch.from_numpy(ref_o.astype(np.float32)), W_UV)
    e = err_rms(out.float().cpu().numpy(), ref)
    note(f"  err vs oracle {e:.3e}")
    assert e <= TOL["bf16"]


def test_fused_step_equals_four_call_step():
    wl = I.workload("v3_b64", B=9)
    case = I.make_case(wl, seq_lens=[1, 64, 65, 700, 1500, 3000, 5000, 8192, 2])
    p = params_for(case, plan=True)
    dc = DeviceCase(case)
    note("fused step vs four-call step")
    a = mla.DecodeStep(p)
    f = mla.DecodeStep(p, fused=True)
    for st in (a, f):
        st(dc.q_nope, dc.q_rope, dc.c_kv, dc.k_pe, dc.kv_scale, dc.block_table, dc.seq_lens, dc.W_UK, dc.W_UV)
    b = f.bind(dc.q_nope, dc.q_rope, dc.c_kv, dc.k_pe, dc.kv_scale, dc.block_table, dc.seq_lens, dc.W_UK, dc.W_UV)
    torch.cuda.synchronize()
    ref_out, ref_lse = f.out.clone(), f.lse.clone()
    f.out.zero_()
    b()
    torch.cuda.synchronize()
    assert torch.equal(a.out, ref_out) and torch.equal(a.lse, ref_lse)
    assert torch.equal(f.out, ref_out)
    ref = O.decode(case)[0]
    assert err_rms(f.out.cpu().numpy(), ref) <= TOL["bf16"]


def test_fused_step_full_size_bitwise():
    """At the bench's decode workload (B=64, lengths U[1024, 8192], balanced splits)
    the fused step reproduces the four-call step bit for bit."""
    wl = I.workload("v3_b64")
    case = I.make_case(wl)
    p = params_for(case, plan=True)
    dc = DeviceCase(case)
    note(f"fused vs four-call at full size: S={p.num_splits} parts={p.num_parts}")
    a = mla.DecodeStep(p)
    f = mla.DecodeStep(p, fused=True)
    for st in (a, f):
        st(dc.q_nope, dc.q_rope, dc.c_kv, dc.k_pe, dc.kv_scale, dc.block_table, dc.seq_lens, dc.W_UK, dc.W_UV)
    torch.cuda.synchronize()
    assert torch.equal(a.out, f.out) and torch.equal(a.lse, f.lse)
