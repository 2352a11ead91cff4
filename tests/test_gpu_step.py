"""The one-call decode step (mla_decode_step) through the C ABI: bit for bit the
output of the separate calls on the same inputs, within tolerance of the oracle,
and its workspace checks."""
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


def run_separate(p, dc, fused):
    st = mla.DecodeStep(p, fused=fused)
    st(dc.q_nope, dc.q_rope, dc.c_kv, dc.k_pe, dc.kv_scale, dc.block_table, dc.seq_lens, dc.W_UK, dc.W_UV)
    return st.out, st.lse


@pytest.mark.parametrize("wl_name,B,lens", [
    ("tiny", 1, None),                              # generic kernels, merge and up-projection apart
    ("v3_b1", 1, None),
    ("v3_b64", 9, [1, 64, 65, 700, 1500, 3000, 5000, 8192, 2]),
    ("v3_sq4_fp8", 3, [4, 700, 4100]),
])
def test_decode_step_equals_separate_calls(wl_name, B, lens):
    wl = I.workload(wl_name, B=B)
    case = I.make_case(wl, seq_lens=lens)
    p = params_for(case, plan=True)
    dc = DeviceCase(case)
    fused = p.latent_dtype == mla.BF16 and p.d_h == 128 and p.d_c == 512 and p.w_dtype == mla.BF16
    note(f"decode_step {wl_name} B={B} lens={case.seq_lens.tolist()} fused_tail={fused}")
    ref_out, ref_lse = run_separate(p, dc, fused)
    n = mla.decode_step_workspace(p)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")     # stale contents: NaN patterns
    out = torch.full_like(ref_out, 7.0)
    lse = torch.full_like(ref_lse, 7.0)
    mla.decode_step(p, dc.q_nope, dc.q_rope, dc.c_kv, dc.k_pe, dc.kv_scale, dc.block_table, dc.seq_lens,
                    dc.W_UK, dc.W_UV, out, lse, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    assert torch.equal(lse, ref_lse)
    ref = O.decode(case)[0]
    e = err_rms(out.float().cpu().numpy(), ref)
    note(f"  err vs oracle {e:.3e}")
    assert e <= TOL[wl.dtype]


def test_decode_step_workspace_checks():
    wl = I.workload("v3_b64", B=2)
    case = I.make_case(wl, seq_lens=[100, 200])
    p = params_for(case, plan=True)
    dc = DeviceCase(case)
    n = mla.decode_step_workspace(p)
    out = torch.empty((2, 1, 128, 128), device="cuda")
    ws = torch.empty(n + 256, dtype=torch.uint8, device="cuda")
    args = (p, dc.q_nope, dc.q_rope, dc.c_kv, dc.k_pe, dc.kv_scale, dc.block_table, dc.seq_lens, dc.W_UK, dc.W_UV, out)
    with pytest.raises(mla.MLAError, match="workspace of"):
        mla.decode_step(*args, None, ws[: n - 1])
    with pytest.raises(mla.MLAError, match="aligned"):
        mla.decode_step(*args, None, ws[8: n + 8])
    mla.decode_step(*args, None, ws[:n])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
