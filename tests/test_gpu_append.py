"""Parity of mla_append_kv (through the C ABI) with the cache-append oracle.

The latent rows and e4m3 codes and scales are integer or copy work: they must
match bit for bit.  The rotated RoPE keys and queries are computed in fp64 on
both sides and rounded once to fp32, then to the storage format; the two fp64
results differ only in the last bits (fused multiply-adds, sin/cos
implementations), so a stored value may differ by one unit in the last place
when it sits on a rounding boundary: the bound is 1 ulp, and the count of such
elements is reported.  Every cache row the append does not own must be left
exactly as it was.
"""
import sys

import numpy as np
import pytest
import torch

from mla_latent_kv_05_amd import inputs as I
from mla_latent_kv_05_amd import mla
from oracle import append as A
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def stored(values, dtype):
    """Exact values -> the storage format: round to fp32, then to dtype."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float64)).float()
    return t if dtype == torch.float32 else t.to(dtype)


def ulps(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """Distance in units in the last place between two same-format tensors."""
    iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return (a.view(iv).to(torch.int64) - b.view(iv).to(torch.int64)).abs()


def tmax(t: torch.Tensor) -> int:
    return int(t.max()) if t.numel() else 0


def check_targets(bt, seq_lens, Sq, num_pages):
    """Host check of the ABI preconditions: every new token's page exists and no
    two new tokens share a cache row."""
    page, slot = A.slots(bt, seq_lens, Sq)
    assert (A.positions(seq_lens, Sq) >= 0).all()
    assert page.min() >= 0 and page.max() < num_pages
    rows = page * 64 + slot
    assert len(np.unique(rows)) == rows.size
    return page, slot


def run_and_check(p, c_kv, k_pe, kv_scale, bt, seq_lens, c_new, kpe_new, q_rope, in_place, offset=0):
    """Append on the GPU and compare every output tensor with the oracle.  With
    `offset`, the device copy of c_new starts `offset` elements into its buffer."""
    B, Sq = p.B, p.Sq
    page, slot = check_targets(bt.numpy(), seq_lens.numpy(), Sq, p.num_pages)
    d = {k: None if v is None else v.cuda().contiguous()
         for k, v in dict(c_kv=c_kv, k_pe=k_pe, kv_scale=kv_scale, bt=bt, sl=seq_lens,
                          kpe_new=kpe_new, q=q_rope).items()}
    buf = torch.zeros(c_new.numel() + offset, dtype=c_new.dtype, device="cuda")
    buf[offset:] = c_new.reshape(-1).cuda()
    d["c_new"] = buf[offset:].view(c_new.shape)
    if offset:
        assert d["c_new"].data_ptr() % 16 != 0
    q_out = None
    if q_rope is not None:
        q_out = d["q"] if in_place else torch.empty_like(d["q"])
    mla.append_kv(p, d["c_new"], d["kpe_new"], d["bt"], d["sl"], d["c_kv"], d["k_pe"], d["kv_scale"],
                  q_rope_in=d["q"], q_rope_out=q_out)
    torch.cuda.synchronize()

    ref = A.append_kv(O.decode_values(c_new), O.decode_values(kpe_new), bt.numpy(), seq_lens.numpy(), Sq,
                      q_rope=None if q_rope is None else O.decode_values(q_rope))
    # latent rows: bit-exact
    if p.kv_dtype == mla.FP8_E4M3:
        exp_c = c_kv.clone()
        exp_c[page, slot] = torch.from_numpy(ref["codes"])
        exp_s = kv_scale.clone()
        exp_s[page, slot] = torch.from_numpy(ref["scales"])
        got_s = d["kv_scale"].cpu()
        assert torch.equal(got_s.view(torch.int32), exp_s.view(torch.int32)), "kv_scale differs"
    else:
        exp_c = c_kv.clone()
        exp_c[page, slot] = stored(ref["c"], c_kv.dtype)
    got_c = d["c_kv"].cpu()
    n_bad = int((got_c != exp_c).sum())
    assert n_bad == 0, f"{n_bad} latent cache elements differ"
    # RoPE keys: the new rows within 1 ulp, every other row untouched
    exp_r = k_pe.clone()
    exp_r[page, slot] = stored(ref["kpe"], k_pe.dtype)
    got_r = d["k_pe"].cpu()
    u = ulps(got_r, exp_r)
    owned = torch.zeros(u.shape[:2], dtype=torch.bool)
    owned[page, slot] = True
    assert tmax(u[~owned]) == 0, "a RoPE-key row the append does not own changed"
    assert tmax(u[owned]) <= 1
    msg = f"k_pe: {int((u[owned] > 0).sum())} of {int(owned.sum()) * k_pe.shape[-1]} at 1 ulp"
    if q_rope is not None:
        uq = ulps(q_out.cpu(), stored(ref["q_rope"], q_rope.dtype))
        assert tmax(uq) <= 1
        msg += f"; q_rope: {int((uq > 0).sum())} of {uq.numel()} at 1 ulp"
    note(msg)


@pytest.mark.parametrize("wl_name,B,Sq,lens,in_place", [
    ("tiny", 3, 3, [3, 70, 128], False),                  # fp32 path; tokens across a page boundary
    ("v3_b64", 64, 1, None, True),                         # the bench's batch, query rotated in place
    ("v3_b64", 3, 2, [2, 100, 4097], True),                # 6 tokens: a wave with 2 of its 4 tokens
    ("v3_sq4_fp8", 8, 4, [4, 63, 64, 65, 127, 128, 4100, 16384], False),   # e4m3 cache
])
def test_append_matches_oracle(wl_name, B, Sq, lens, in_place):
    wl = I.workload(wl_name, B=B, Sq=Sq)
    case = I.make_case(wl, seq_lens=lens)
    f32 = wl.dtype == "f32"
    fl = mla.F32 if f32 else mla.BF16
    kv = mla.FP8_E4M3 if wl.dtype == "fp8" else fl
    p = mla.make_params(B, Sq, wl.H, wl.d_h, wl.d_c, wl.d_r, case.num_pages, case.max_pages, scale=wl.scale,
                        q_dtype=fl, w_dtype=fl, kv_dtype=kv, pe_dtype=fl, latent_dtype=fl)
    c_new, kpe_new = I.random_new_tokens(wl, seed=7000 + B)
    note(f"append {wl_name} B={B} Sq={Sq} kv={kv} in_place={in_place}")
    run_and_check(p, case.c_kv, case.k_pe, case.kv_scale, case.block_table, case.seq_lens, c_new, kpe_new,
                  case.q_rope, in_place)


@pytest.mark.parametrize("d_c,d_r,offset", [(60, 10, 0), (64, 16, 1)])
def test_append_scalar_path(d_c, d_r, offset):
    """A latent width that is not a multiple of 8, and a latent input that is not
    16-byte aligned, take the one-value-per-lane path."""
    wl = I.workload("tiny", B=3, Sq=2, d_c=d_c, d_r=d_r, dtype="bf16")
    case = I.make_case(wl, seq_lens=[2, 64, 129])
    p = mla.make_params(wl.B, wl.Sq, wl.H, wl.d_h, d_c, d_r, case.num_pages, case.max_pages, scale=wl.scale)
    c_new, kpe_new = I.random_new_tokens(wl, seed=7300 + d_c)
    note(f"append scalar path d_c={d_c} d_r={d_r} offset={offset}")
    run_and_check(p, case.c_kv, case.k_pe, None, case.block_table, case.seq_lens, c_new, kpe_new,
                  case.q_rope, in_place=True, offset=offset)


def sparse_cache(lens, Sq, d_c, d_r, dtype, seed=11):
    """A small cache whose pages serve only the new tokens: the block table is as
    wide as the longest sequence needs, with -1 everywhere else (an append reads
    only the entries of its tokens' pages)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    max_pages = int((lens.max() + 63) // 64)
    bt = np.full((len(lens), max_pages), -1, dtype=np.int32)
    need = sorted({(b, int(t) // 64) for b in range(len(lens)) for t in range(lens[b] - Sq, lens[b])})
    perm = rng.permutation(len(need) + 2)              # two extra pages nobody owns
    for k, (b, j) in enumerate(need):
        bt[b, j] = perm[k]
    P = len(need) + 2
    c = torch.from_numpy(rng.standard_normal((P, 64, d_c), dtype=np.float32)).to(dtype)
    r = torch.from_numpy(rng.standard_normal((P, 64, d_r), dtype=np.float32)).to(dtype)
    return torch.from_numpy(bt), torch.from_numpy(lens.astype(np.int32)), c, r


@pytest.mark.parametrize("q_fmt", ["bf16", "f32"])
def test_append_long_positions(q_fmt):
    """Positions up to 131071 (angles up to 1.3e5 rad): bf16 cache, activations in
    bf16 or fp32 (fp32 latent rows are rounded to bf16 on the way in)."""
    lens, Sq, H = [131072, 65540, 4, 100000], 4, 128
    bt, sl, c_kv, k_pe = sparse_cache(lens, Sq, 512, 64, torch.bfloat16)
    wl = I.workload("v3_b64", B=len(lens), Sq=Sq)
    c_new, kpe_new = I.random_new_tokens(wl, seed=8100, fmt=q_fmt)
    qd = mla.F32 if q_fmt == "f32" else mla.BF16
    q = torch.from_numpy(np.random.default_rng(8101).standard_normal((len(lens), Sq, H, 64),
                                                                    dtype=np.float32)).to(c_new.dtype)
    p = mla.make_params(len(lens), Sq, H, 128, 512, 64, c_kv.shape[0], bt.shape[1], q_dtype=qd,
                        kv_dtype=mla.BF16, pe_dtype=mla.BF16)
    note(f"append long positions q_fmt={q_fmt}")
    run_and_check(p, c_kv, k_pe, None, bt, sl, c_new, kpe_new, q, in_place=False)


def test_append_then_decode_reads_the_new_tokens():
    """Appending the last Sq tokens of every sequence and then decoding gives the
    oracle's attention over the cache that holds them (the append's rows are what
    the decode reads)."""
    wl = I.workload("v3_b64", B=6, Sq=2)
    case = I.make_case(wl, seq_lens=[2, 65, 130, 640, 1000, 2049])
    # drawn like the rest of the cache (standard normal), the distribution the
    # decode tolerance is set for
    c_new, kpe_new = I.random_new_tokens(wl, seed=8200, latent_std=1.0)
    p = mla.make_params(wl.B, wl.Sq, wl.H, wl.d_h, wl.d_c, wl.d_r, case.num_pages, case.max_pages, scale=wl.scale)
    d_c, d_r = case.c_kv.cuda(), case.k_pe.cuda()
    bt, sl = case.block_table.cuda(), case.seq_lens.cuda()
    check_targets(case.block_table.numpy(), case.seq_lens.numpy(), wl.Sq, case.num_pages)
    note("append then decode")
    mla.append_kv(p, c_new.cuda(), kpe_new.cuda(), bt, sl, d_c, d_r)
    st = mla.DecodeStep(p)
    st(case.q_nope.cuda(), case.q_rope.cuda(), d_c, d_r, None, bt, sl, case.W_UK.cuda(), case.W_UV.cuda())
    torch.cuda.synchronize()
    # oracle: the same cache with the appended rows written by the append oracle
    ref = A.append_kv(O.decode_values(c_new), O.decode_values(kpe_new), case.block_table.numpy(),
                      case.seq_lens.numpy(), wl.Sq)
    page, slot = ref["page"], ref["slot"]
    c2, r2 = case.c_kv.clone(), case.k_pe.clone()
    c2[page, slot] = stored(ref["c"], c2.dtype)
    r2[page, slot] = stored(ref["kpe"], r2.dtype)
    case2 = I.Case(wl=wl, seq_lens=case.seq_lens, block_table=case.block_table, c_kv=c2, kv_scale=None,
                   k_pe=r2, q_nope=case.q_nope, q_rope=case.q_rope, W_UK=case.W_UK, W_UV=case.W_UV)
    out_ref = O.decode(case2)[0]
    got = st.out.cpu().double().numpy()
    ref_out = np.asarray(out_ref, dtype=np.float64).reshape(got.shape)
    err = float(np.max(np.abs(got - ref_out))) / float(np.sqrt(np.mean(ref_out ** 2)))
    note(f"append+decode err {err:.3e}")
    assert err <= 2e-2
