"""Parity of the non-absorbed path (mla_decompress_kv, mla_prefill_attention)
with the oracles, through the C ABI.

Decompressed keys and values: every element within bf16 rounding of the fp64
product.  Attention: for every row, max|gpu - oracle| / RMS(oracle row) <= 2e-2
(bf16 keys, values and weights), the oracle being the decode oracle with Sq = the
number of new tokens (it applies the causal rule to every row), which the oracle
tests pin to the non-absorbed definition.  The error is taken per row because the
rows see from one to thousands of positions: a row that sees one position returns
that position's value row (bf16-rounded), whose size is that of a single value,
while rows averaging many positions are smaller.  Rows that see nothing are 0
exactly.  Decompressed positions from seq_len to the next multiple of 256 are
zeros and later ones are never written.
"""
import sys

import numpy as np
import pytest
import torch

from mla_latent_kv_05_amd import inputs as I
from mla_latent_kv_05_amd import mla
from oracle import oracle as O
from oracle import prefill as PF
from tests.helpers import assert_bf16_rounding, err_rows

pytestmark = pytest.mark.gpu

SENT = -12288.0     # bf16-exact sentinel of untouched outputs


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def validate(case):
    lens = case.seq_lens.to(torch.int64)
    assert int(lens.max()) <= case.max_pages * 64
    for b in range(case.wl.B):
        n = -(-int(lens[b]) // 64)
        if n:
            ids = case.block_table[b, :n]
            assert int(ids.min()) >= 0 and int(ids.max()) < case.num_pages


def params(case, **kw):
    wl = case.wl
    return mla.make_params(wl.B, wl.Sq, wl.H, wl.d_h, wl.d_c, wl.d_r, case.num_pages, case.max_pages,
                           scale=wl.scale, **kw)


def run_path(case, p):
    """decompress + attention on the GPU; returns (k_nope, v_t, out) on the CPU."""
    wl = case.wl
    validate(case)
    L = mla.lmax(p)
    kn = torch.full((wl.B, L, wl.H, wl.d_h), SENT, dtype=torch.bfloat16, device="cuda")
    vt = torch.full((wl.B, wl.H, wl.d_h, L), SENT, dtype=torch.bfloat16, device="cuda")
    out = torch.empty((wl.B, wl.Sq, wl.H, wl.d_h), dtype=torch.float32 if p.out_dtype == mla.F32 else torch.bfloat16,
                      device="cuda")
    d = {k: getattr(case, k).cuda() for k in ("c_kv", "k_pe", "block_table", "seq_lens", "W_UK", "W_UV",
                                              "q_nope", "q_rope")}
    mla.decompress_kv(p, d["c_kv"], d["block_table"], d["seq_lens"], d["W_UK"], d["W_UV"], kn, vt)
    mla.prefill_attention(p, d["q_nope"], d["q_rope"], kn, vt, d["k_pe"], d["block_table"], d["seq_lens"], out)
    torch.cuda.synchronize()
    return kn.cpu(), vt.cpu(), out.cpu()


def check_decompressed(case, kn, vt):
    wl = case.wl
    c = O.cache_values(case)
    wuk, wuv = O.decode_values(case.W_UK), O.decode_values(case.W_UV)
    knd = kn.double().numpy()
    vtd = vt.double().numpy()
    for b in range(wl.B):
        L = int(case.seq_lens[b])
        if L > 0:
            K, V = PF.decompress_kv(PF.sequence_latents(c, case.block_table.numpy()[b], L), wuk, wuv)
            assert_bf16_rounding(knd[b, :L], K, acc_rel=1e-4)
            assert_bf16_rounding(vtd[b, :, :, :L], V.transpose(1, 2, 0), acc_rel=1e-4)
        Lz = -(-L // 256) * 256
        assert (knd[b, L:Lz] == 0).all() and (vtd[b, :, :, L:Lz] == 0).all()
        assert (knd[b, Lz:] == SENT).all() and (vtd[b, :, :, Lz:] == SENT).all()


@pytest.mark.parametrize("B,Sq,lens", [
    (2, 96, [200, 96]),            # a cached prefix, and a whole-prompt prefill
    (3, 70, [70, 133, 64]),        # new tokens not a multiple of 32 / 128; one tile past a page
    (1, 160, [1000]),              # two query blocks over a long prefix
])
def test_prefill_path_matches_oracle(B, Sq, lens):
    wl = I.workload("v3_b64", B=B, Sq=Sq)
    case = I.make_case(wl, seq_lens=lens)
    p = params(case)
    assert mla.prefer_absorbed(p) == (Sq < 120)     # the switch (these cases run the non-absorbed path anyway)
    note(f"prefill B={B} Sq={Sq} lens={lens}")
    kn, vt, out = run_path(case, p)
    check_decompressed(case, kn, vt)
    ref = O.decode(case)[0]
    err = err_rows(out.double().numpy(), ref)
    note(f"prefill err {err:.3e}")
    assert err <= 2e-2


def test_prefill_rows_with_nothing_visible():
    """seq_len below the number of new tokens: the first rows see nothing (output 0)."""
    wl = I.workload("v3_b64", B=2, Sq=64)
    case = I.make_case(wl, seq_lens=[40, 64])
    p = params(case)
    note("prefill degenerate rows")
    _, _, out = run_path(case, p)
    ref = O.decode(case)[0]
    assert (out[0, :24] == 0).all()
    assert err_rows(out.double().numpy(), ref) <= 2e-2


@pytest.mark.parametrize("Sq,lens", [(16, [16, 300, 777]), (64, [64, 200, 1000])])
def test_both_paths_agree_where_both_apply(Sq, lens):
    """Where both paths take the new tokens, the absorbed steps and the non-absorbed
    path agree with each other and with the oracle."""
    wl = I.workload("v3_b64", B=3, Sq=Sq)
    case = I.make_case(wl, seq_lens=lens)
    p = params(case)
    note(f"absorbed vs non-absorbed at Sq={Sq}")
    _, _, out_na = run_path(case, p)
    d = {k: getattr(case, k).cuda() for k in ("q_nope", "q_rope", "c_kv", "k_pe", "block_table", "seq_lens",
                                              "W_UK", "W_UV")}
    st = mla.DecodeStep(p)
    st(d["q_nope"], d["q_rope"], d["c_kv"], d["k_pe"], None, d["block_table"], d["seq_lens"], d["W_UK"], d["W_UV"])
    torch.cuda.synchronize()
    ref = O.decode(case)[0]
    e_na = err_rows(out_na.double().numpy(), ref)
    e_ab = err_rows(st.out.cpu().double().numpy(), ref)
    note(f"non-absorbed err {e_na:.3e}, absorbed err {e_ab:.3e}")
    assert e_na <= 2e-2 and e_ab <= 2e-2
    # each within 2e-2 of the oracle per row, hence within 4e-2 of each other
    assert err_rows(out_na.double().numpy(), st.out.cpu().double().numpy()) <= 4e-2


def test_empty_sequence_and_prefix_only_rows():
    """A sequence of length 0 next to normal ones: nothing of it is written and all
    its rows are 0; the others are unaffected."""
    wl = I.workload("v3_b64", B=3, Sq=40)
    case = I.make_case(wl, seq_lens=[0, 40, 300])
    p = params(case)
    note("prefill with an empty sequence")
    kn, vt, out = run_path(case, p)
    check_decompressed(case, kn, vt)
    assert (out[0] == 0).all()
    ref = O.decode(case)[0]
    assert err_rows(out[1:].double().numpy(), ref[1:]) <= 2e-2


def test_full_size_sampled():
    """The bench's workload (4 sequences x 4,096 new tokens, whole-prompt prefill) in
    its launch configuration, bf16 output; decompressed rows and outputs checked on
    sampled positions and rows that the oracle computes one by one."""
    B, x = 4, 4096
    wl = I.workload("v3_b64", B=B, Sq=x)
    note("prefill full size: generating")
    case = I.make_case(wl, seq_lens=[x] * B)
    p = params(case, out_dtype=mla.BF16)
    validate(case)
    L = mla.lmax(p)
    d = {k: getattr(case, k).cuda() for k in ("c_kv", "k_pe", "block_table", "seq_lens", "W_UK", "W_UV",
                                              "q_nope", "q_rope")}
    kn = torch.empty((B, L, wl.H, wl.d_h), dtype=torch.bfloat16, device="cuda")
    vt = torch.empty((B, wl.H, wl.d_h, L), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, x, wl.H, wl.d_h), dtype=torch.bfloat16, device="cuda")
    note("prefill full size: running")
    mla.decompress_kv(p, d["c_kv"], d["block_table"], d["seq_lens"], d["W_UK"], d["W_UV"], kn, vt)
    mla.prefill_attention(p, d["q_nope"], d["q_rope"], kn, vt, d["k_pe"], d["block_table"], d["seq_lens"], out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    # decompressed rows: first, last and random positions of every sequence
    c = O.cache_values(case)
    wuk, wuv = O.decode_values(case.W_UK), O.decode_values(case.W_UV)
    bt = case.block_table.numpy()
    for b in range(B):
        pos = np.unique(np.concatenate([[0, x - 1], rng.integers(0, x, 6)]))
        lat = c[bt[b, pos // 64], pos % 64]
        K, V = PF.decompress_kv(lat, wuk, wuv)
        assert_bf16_rounding(kn[b, pos].double().cpu().numpy(), K, acc_rel=1e-4)
        assert_bf16_rounding(vt[b][:, :, pos].double().cpu().numpy(), V.transpose(1, 2, 0), acc_rel=1e-4)
    # outputs: the first and last new tokens and random ones, first/last/random heads
    toks = np.unique(np.concatenate([[0, 1, x - 1], rng.integers(0, x, 5)]))
    heads = np.unique(np.concatenate([[0, wl.H - 1], rng.integers(0, wl.H, 2)]))
    rows = np.array([(b * x + s) * wl.H + h for b in range(B) for s in toks for h in heads], dtype=np.int64)
    note(f"prefill full size: oracle on {len(rows)} rows")
    ref = O.decode(case, rows=rows)[0]
    got = out.float().cpu().numpy().reshape(-1, wl.d_h)[rows]
    e = err_rows(got, ref, out_bf16=True)
    note(f"prefill full size err {e:.3e}")
    assert e <= 2e-2
