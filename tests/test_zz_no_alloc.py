"""mla_decode_step_noalloc through the C ABI: the same output as mla_decode_step
(with a caller workspace) on two calls in a row, the second on a smaller batch,
the static scratch keeping the first call's contents in between."""
import ctypes
import sys

import pytest
import torch

from mla_latent_kv_05_amd import inputs as I
from mla_latent_kv_05_amd import mla
from tests.helpers import DeviceCase, params_for

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def step_args(p, dc, out, lse):
    return (ctypes.byref(p), *(ctypes.c_void_p(t.data_ptr()) if t is not None else None
                                for t in (dc.q_nope, dc.q_rope, dc.c_kv, dc.k_pe, dc.kv_scale, dc.block_table,
                                          dc.seq_lens, dc.W_UK, dc.W_UV, out, lse)))


@pytest.mark.parametrize("first,second", [
    (("v3_b64", [1, 64, 65, 700, 1500, 3000, 5000, 8192, 2]), ("v3_b64", [300, 4100, 9])),
    (("v3_sq4_fp8", [4, 700, 4100, 2000]), ("v3_sq4_fp8", [129])),
    (("v3_b1", None), ("tiny", None)),
])
def test_noalloc_step_matches_workspace_step(first, second):
    L = mla.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for name, lens in (first, second):
        wl = I.workload(name, B=1 if lens is None else len(lens))
        case = I.make_case(wl, seq_lens=lens)
        p = params_for(case, plan=True)
        dc = DeviceCase(case)
        note(f"noalloc {name} lens={case.seq_lens.tolist()} workspace={mla.decode_step_workspace(p)}")
        rows = (p.B, p.Sq, p.H)
        td = torch.float32 if p.out_dtype == mla.F32 else torch.bfloat16
        ref = torch.full(rows + (p.d_h,), 7.0, dtype=td, device="cuda")
        ref_lse = torch.full(rows, 7.0, device="cuda")
        ws = torch.full((mla.decode_step_workspace(p),), 0xFF, dtype=torch.uint8, device="cuda")
        args = step_args(p, dc, ref, ref_lse)
        assert L.mla_decode_step(*args, ctypes.c_void_p(ws.data_ptr()), ws.numel(), st) == 0, \
            L.mla_last_error().decode()
        out = torch.full_like(ref, -3.0)
        lse = torch.full_like(ref_lse, -3.0)
        assert L.mla_decode_step_noalloc(*step_args(p, dc, out, lse), st) == 0, L.mla_last_error().decode()
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all()
        assert torch.equal(out, ref)
        assert torch.equal(lse, ref_lse)
