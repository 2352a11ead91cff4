"""Benchmark of one absorbed-MLA decode step on one MI355X.

A step = mla_absorb_q + mla_decode_splitkv + mla_combine_lse + mla_up_v over
the whole batch (one layer), on synthetic seeded inputs already resident in
HBM; the same step with the last two calls fused (mla_combine_up_v, bit for bit
the same output) is timed as well, and `value` is the faster of the two.  Default workload: B=64 sequences, lengths uniform in [1024, 8192],
DeepSeek-V3 head shapes (H=128, d_h=128, d_c=512, d_r=64), bf16, pages of 64
tokens in a randomly permuted block table, Sq=1.

The inputs are replicated in HBM (by default enough replicas to hold at least
1 GiB, at least 4) and the steps rotate over the replicas, so the 256 MB
last-level cache cannot serve one step from the previous one.

Timing, in this order:
  1. the step with the fused tail: untimed warm-up steps (at least W, then blocks
     of WARM_BLOCK steps, each followed by a synchronize, for WARM_S seconds),
     then exactly K timed steps bracketed by a synchronize and events (events
     only at block boundaries);
  2. the same for the four-call step;
  3. the attention kernel alone (the roofline object): a fixed warm-up of
     KERNEL_WARMUP launches, then max(KERNEL_LAUNCHES, K) launches back to back
     on the launch stream inside one event pair, whatever --steps is.
The GPU reaches its sustained step rate only after some hundreds of steps of
load (measured at 64 x 4,096 positions: 5 warm-up steps then 20 timed ones read
~10% slower than after 300 more, and still ~2% slower than after 1,000 more), so
each route gets WARM_S seconds of warm-up steps whatever W is; the JSON gives W
and the warm-up steps each route ran.  The warm-up synchronizes every WARM_BLOCK
steps, as a decode loop does to read each step's result: thousands of steps
enqueued at once (a second of work) left the next timed steps 5-20 % slower for a
while, the GPU's power management having lowered its clocks.
The oracle leg (cpu_baseline) also compares the step's output for the sequences
it computed with the GPU step's output (max and RMS error over the output RMS).

Prints one JSON line.  value = latent-cache TB/s = (tokens x 1152 B) / step time.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
STEP_BLOCK = 50                # steps per block of the step-time spread
WARM_S = 0.5                   # seconds of warm-up steps per route (at least W steps)
WARM_BLOCK = 50                # warm-up steps between synchronizes
KERNEL_WARMUP = 300            # untimed attention launches before the kernel leg
KERNEL_LAUNCHES = 600          # timed attention launches (at least; more when K is larger)
REPLICA_BYTES = 1 << 30        # inputs replicated until the replicas hold this many bytes


def pct(xs):
    """[p10, p50, p90] of a list of times, rounded to 0.01."""
    import numpy as np
    return [round(float(v), 2) for v in np.percentile(np.asarray(xs, dtype=np.float64), [10, 50, 90])]


# rocprofv3 counter summary of the attention kernel on this workload (FETCH_SIZE /
# WRITE_SIZE in KiB per dispatch) and the hash of the kernel source it was taken on
COUNTERS = os.path.join(ROOT, "profiles", "decode128_bf16_v3_b64_counters.txt")
# the sources of the attention kernel the counters were taken on
KERNEL_SRCS = [os.path.join(ROOT, "mla_latent_kv_05_amd", "csrc", f)
               for f in ("kernels_decode128.hip", "decode_common.h", "gfx950.h", "mla_internal.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="v3_b64")
    ap.add_argument("--replicas", type=int, default=0, help="input replicas (0: enough for 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-reps", type=int, default=10)
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a device copy of this size (for scaling HBM counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mla_latent_kv_05_amd import accounting as A
    from mla_latent_kv_05_amd import inputs as I
    from mla_latent_kv_05_amd import mla

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)
    wl = I.workload(args.workload)
    case = I.make_case(wl)
    lens = case.seq_lens.tolist()
    fl = mla.F32 if wl.dtype == "f32" else mla.BF16
    kv = mla.FP8_E4M3 if wl.dtype == "fp8" else fl
    # bf16 partials with a bf16 latent: half the bytes the attention writes and the
    # merge reads (each partial row rounded once, as o_latent is); the planner sizes
    # the parts for them
    # an e4m3 cache holds power-of-two token scales (the append's format, which the
    # generator follows): MLA_FLAG_POW2_SCALE lets the kernel widen with one
    # instruction per two codes
    p = mla.make_params(wl.B, wl.Sq, wl.H, wl.d_h, wl.d_c, wl.d_r, case.num_pages, case.max_pages,
                        scale=wl.scale, q_dtype=fl, w_dtype=fl, kv_dtype=kv, pe_dtype=fl,
                        latent_dtype=fl, out_dtype=mla.F32, part_dtype=mla.F32 if wl.dtype == "f32" else mla.BF16,
                        flags=mla.FLAG_POW2_SCALE if wl.dtype == "fp8" else 0)
    p = mla.plan_splits(p, max(lens), case.total_tokens, num_cus=props.multi_processor_count,
                        min_splits=wl.min_splits)

    names = ("q_nope", "q_rope", "c_kv", "k_pe", "kv_scale", "block_table", "seq_lens", "W_UK", "W_UV")
    base = {k: (None if getattr(case, k) is None else getattr(case, k).to(dev)) for k in names}
    rep_bytes = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    if args.replicas < 1:
        args.replicas = max(4, min(256, -(-REPLICA_BYTES // rep_bytes)))
    reps = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()}
                     for _ in range(args.replicas - 1)]
    step = mla.DecodeStep(p, device=dev)
    stream = torch.cuda.current_stream()

    # each replica's four calls, marshalled once (the library still checks its
    # arguments on every call)
    bound = [step.bind(t["q_nope"], t["q_rope"], t["c_kv"], t["k_pe"], t["kv_scale"], t["block_table"],
                       t["seq_lens"], t["W_UK"], t["W_UV"], stream) for t in reps]

    def run(r):
        b = bound[r]
        b.absorb_q()
        b.decode_splitkv()
        b.combine_lse()
        b.up_v()

    # the step with the fused tail (merge + up-projection in one launch): same output
    step_f = mla.DecodeStep(p, device=dev, fused=True)
    bound_f = [step_f.bind(t["q_nope"], t["q_rope"], t["c_kv"], t["k_pe"], t["kv_scale"], t["block_table"],
                           t["seq_lens"], t["W_UK"], t["W_UV"], stream) for t in reps]

    def warm(step_fn, seconds=WARM_S):
        """W warm-up steps, then blocks of WARM_BLOCK steps, each followed by a
        synchronize (as a decode loop synchronizes to read each step's result),
        until `seconds` have passed; returns the number of warm-up steps."""
        for i in range(args.warmup):
            step_fn(i)
        torch.cuda.synchronize()
        n, t0 = args.warmup, time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for i in range(WARM_BLOCK):
                step_fn(i)
            torch.cuda.synchronize()
            n += WARM_BLOCK
        return n

    warm_runs = {}

    # 1. the fused step: warm-up steps, then exactly K timed steps bracketed by a
    # synchronize and events; an event at every block boundary (one per STEP_BLOCK
    # steps) gives the spread of the per-step time without gaps inside the steps
    # (the output checks run after the timed steps: the first allocation of a device
    # block by torch between the warm-up and the timed steps slowed the next steps
    # by 10-20 % for about a millisecond)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(-(-args.steps // STEP_BLOCK) + 1)]
    warm_runs["fused_tail"] = warm(lambda i: bound_f[i % args.replicas]())
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    marks[0].record(stream)
    for i in range(args.steps):
        bound_f[i % args.replicas]()
        if (i + 1) % STEP_BLOCK == 0 or i + 1 == args.steps:
            marks[-(-(i + 1) // STEP_BLOCK)].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_fused = marks[0].elapsed_time(marks[-1]) / args.steps
    blk_us = [marks[k].elapsed_time(marks[k + 1]) * 1e3 / min(STEP_BLOCK, args.steps - k * STEP_BLOCK)
              for k in range(len(marks) - 1)]

    assert torch.isfinite(step_f.out).all(), "non-finite output"

    # 2. the four-call step, the same way (events around the whole loop only)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    warm_runs["four_calls"] = warm(lambda i: run(i % args.replicas))
    t_start.record(stream)
    for i in range(args.steps):
        run(i % args.replicas)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    assert torch.equal(step_f.out, step.out), "fused tail differs from the four-call step"

    # e4m3 cache: also the route that expands the cache to bf16 first (for a step
    # bound by the matrix cores); same result within the e4m3 bound
    ms_expand = None
    if wl.dtype == "fp8":
        step_e = mla.DecodeStep(p, device=dev, fused=True, expand=True)
        bound_e = [step_e.bind(t["q_nope"], t["q_rope"], t["c_kv"], t["k_pe"], t["kv_scale"], t["block_table"],
                               t["seq_lens"], t["W_UK"], t["W_UV"], stream) for t in reps]
        x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        warm_runs["expand_fused_tail"] = warm(lambda i: bound_e[i % args.replicas]())
        x0.record(stream)
        for i in range(args.steps):
            bound_e[i % args.replicas]()
        x1.record(stream)
        torch.cuda.synchronize()
        ms_expand = x0.elapsed_time(x1) / args.steps
        diff = float((step_e.out - step.out).abs().max() / step.out.pow(2).mean().sqrt())
        assert diff <= 6e-2, f"expanded-cache route differs from the e4m3 route by {diff}"

    # a small batch of single new tokens at a short context (where the planner itself
    # takes one-page splits): also the single-launch step, for reference (not a
    # headline route: slower on this GPU; equal within rounding, not bit for bit).  Its
    # attention items are single pages, so at long contexts it is not a route at all.
    ms_single = None
    L = mla.lib()
    if (L.mla_decode_step_persistent_workspace(ctypes.byref(p)) > 0
            and L.mla_decode_kernel_name(ctypes.byref(p)) == b"page_bf16"):
        nws = mla.decode_step_persistent_workspace(p)
        ws1 = [torch.zeros(nws, dtype=torch.uint8, device=dev) for _ in reps]
        out1 = torch.empty_like(step.out)
        ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        args1 = [(ctypes.byref(p), ptr(t["q_nope"]), ptr(t["q_rope"]), ptr(t["c_kv"]), ptr(t["k_pe"]),
                  ptr(t["block_table"]), ptr(t["seq_lens"]), ptr(t["W_UK"]), ptr(t["W_UV"]), ptr(out1), None,
                  ptr(ws1[r]), ctypes.c_int64(nws), ctypes.c_void_p(stream.cuda_stream)) for r, t in enumerate(reps)]
        fn1 = L.mla_decode_step_persistent

        def single(i):
            st = fn1(*args1[i % args.replicas])
            if st != 0:
                raise mla.MLAError(st, L.mla_last_error().decode())

        warm_runs["single_launch"] = warm(single)
        u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        u0.record(stream)
        for i in range(args.steps):
            single(i)
        u1.record(stream)
        torch.cuda.synchronize()
        ms_single = u0.elapsed_time(u1) / args.steps
        single(0)                                  # the replicas hold the same inputs
        torch.cuda.synchronize()
        diff = float((out1.float() - step_f.out.float()).abs().max() / step_f.out.float().pow(2).mean().sqrt())
        assert diff <= 2e-2, f"single-launch step differs from the fused step by {diff}"
        assert mla.device_errors() == 0, "single-launch step: device error word set"

    cost = A.step_cost(wl.B, wl.Sq, wl.H, wl.d_h, wl.d_c, wl.d_r, lens, fmt=wl.dtype, out_fmt="f32")
    ms_four = ms_step
    ms_step = min(ms_step, ms_fused)               # the headline step: the fastest route (same result)
    expand_wins = ms_expand is not None and ms_expand < ms_step
    if expand_wins:
        ms_step = ms_expand
    # the attention launch of the headline route (on the expanded bf16 copy when the
    # expanding route is the fastest)
    dec_calls = [b.decode_splitkv for b in (bound_e if expand_wins else bound)]

    # 3. the attention kernel alone: fixed warm-up, then back-to-back launches inside
    # one event pair on the launch stream (no per-launch events, whose stream gaps
    # would be timed too); events at block boundaries give the spread
    n_dec = max(KERNEL_LAUNCHES, args.steps)
    kmarks = [torch.cuda.Event(enable_timing=True) for _ in range(-(-n_dec // STEP_BLOCK) + 1)]
    for i in range(KERNEL_WARMUP):
        dec_calls[i % args.replicas]()
    torch.cuda.synchronize()
    kmarks[0].record(stream)
    for i in range(n_dec):
        dec_calls[i % args.replicas]()
        if (i + 1) % STEP_BLOCK == 0 or i + 1 == n_dec:
            kmarks[-(-(i + 1) // STEP_BLOCK)].record(stream)
    torch.cuda.synchronize()
    dec_avg_ms = kmarks[0].elapsed_time(kmarks[-1]) / n_dec
    dec_blk_us = [kmarks[k].elapsed_time(kmarks[k + 1]) * 1e3 / min(STEP_BLOCK, n_dec - k * STEP_BLOCK)
                  for k in range(len(kmarks) - 1)]

    assert dec_avg_ms <= ms_step, (f"attention launch {dec_avg_ms * 1e3:.2f} us exceeds the step "
                                   f"{ms_step * 1e3:.2f} us it is part of")
    tb_s = cost.cache_bytes / (ms_step * 1e-3) / 1e12
    achieved_gbs = cost.decode_bytes / (dec_avg_ms * 1e-3) / 1e9
    achieved_tflops = cost.decode_flops / (dec_avg_ms * 1e-3) / 1e12
    # the attention kernel's bound: HBM or the bf16 matrix cores, whichever takes longer
    mfma_bound = cost.decode_flops / (BF16_PEAK_TFLOPS * 1e12) > cost.decode_bytes / (HBM_PEAK_GBS * 1e9)
    roofline_us = max(cost.total_bytes / (HBM_PEAK_GBS * 1e9), cost.flops / (BF16_PEAK_TFLOPS * 1e12)) * 1e6

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    peaks = measured_peaks(dev, stream)
    append = append_bench(mla, A, wl, p, reps[0], dev, stream, args)
    prefill = None if args.no_prefill else prefill_bench(mla, A, dev, stream, args)
    if prefill is not None:
        for k in ("decompress", "attention", "path"):
            prefill[k]["frac_of_measured_gemm"] = round(prefill[k]["achieved"] / peaks["bf16_gemm_tflops"], 4)

    cpu = parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(case, args.cpu_budget_s, step_f.out.float().cpu().numpy())

    result = {
        "metric": "MLA absorbed decode µs/step + latent-cache TB/s at B=64, L=4096, bf16",
        "value": round(tb_s, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_runs,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype != "f32" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"absorbed MLA decode, B={wl.B}, Sq={wl.Sq}, H={wl.H}, d_h={wl.d_h}, "
                        f"d_c={wl.d_c}, d_r={wl.d_r}, seq_lens U[{wl.seq_lo},{wl.seq_hi}] "
                        f"(sum {case.total_tokens}), page 64, permuted pages, {wl.dtype} cache",
            "name": wl.name, "B": wl.B, "Sq": wl.Sq, "tokens": case.total_tokens,
            "num_splits": p.num_splits, "num_parts": p.num_parts,
            "partials": "bf16" if p.part_dtype == mla.BF16 else "f32",
            "decode_kernel": mla.decode_kernel_name(p), "replicas": args.replicas,
        },
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm",
            "kernel": "mla_decode_splitkv" + (" (on the expanded bf16 copy)" if expand_wins else ""),
            "achieved": round(achieved_tflops, 1) if mfma_bound else round(achieved_gbs, 1),
            "peak": BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s",
            "frac": round(achieved_tflops / BF16_PEAK_TFLOPS if mfma_bound else achieved_gbs / HBM_PEAK_GBS, 4),
            "hbm_gbs": round(achieved_gbs, 1),
            "traffic": measured_traffic(wl.name),
            "launch_us": round(dec_avg_ms * 1e3, 2),
            "launches_timed": n_dec,
            "block_us_p10_p50_p90": pct(dec_blk_us), "block_launches": STEP_BLOCK,
            "bytes_per_launch": cost.decode_bytes,
            "mfma_tflops": round(cost.decode_flops / (dec_avg_ms * 1e-3) / 1e12, 1),
            "frac_of_measured_copy": round(achieved_gbs / peaks["hbm_copy_gbs"], 4),
        },
        "measured_peaks": peaks,
        "step_roofline": {"bytes": cost.total_bytes, "flops": cost.flops, "t_roof_us": round(roofline_us, 2),
                          "frac": round(roofline_us / (ms_step * 1e3), 4)},
        "steps_timed": {
            "four_calls": {"calls": "absorb_q, decode_splitkv, combine_lse, up_v",
                           "us_per_step": round(ms_four * 1e3, 2),
                           "value": round(cost.cache_bytes / (ms_four * 1e-3) / 1e12, 4)},
            "fused_tail": {"calls": "absorb_q, decode_splitkv, combine_up_v",
                           "us_per_step": round(ms_fused * 1e3, 2),
                           "value": round(cost.cache_bytes / (ms_fused * 1e-3) / 1e12, 4),
                           "block_us_p10_p50_p90": pct(blk_us), "block_steps": STEP_BLOCK},
            **({"expand_fused_tail": {"calls": "expand_kv, absorb_q, decode_splitkv (bf16 copy), combine_up_v",
                                      "us_per_step": round(ms_expand * 1e3, 2),
                                      "value": round(cost.cache_bytes / (ms_expand * 1e-3) / 1e12, 4)}}
               if ms_expand is not None else {}),
            **({"single_launch": {"calls": "decode_step_persistent (one launch; reference, not a headline route)",
                                  "us_per_step": round(ms_single * 1e3, 2),
                                  "value": round(cost.cache_bytes / (ms_single * 1e-3) / 1e12, 4)}}
               if ms_single is not None else {}),
        },
        "append": append,
        "prefill": prefill,
        "cpu_baseline": cpu,
        "parity": parity,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(result), flush=True)


def measured_peaks(dev, stream):
    """Practical peaks on this GPU, as context for the spec peaks: a 1 GiB device copy
    (bytes read + written per second) and a large bf16 matrix product (torch's
    library GEMM, contiguous operands)."""
    import numpy as np
    import torch

    def timed(fn, n):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3

    src = torch.ones(1 << 28, device=dev)             # 1 GiB of fp32
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 10)
    del src, dst
    n = 8192
    a = torch.randn((n, n), device=dev).bfloat16()
    b = torch.randn((n, n), device=dev).bfloat16()
    t_mm = timed(lambda: torch.mm(a, b), 10)
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_copy_gbs": round(2 * (1 << 30) / t_copy / 1e9, 1),
            "bf16_gemm_tflops": round(2 * n ** 3 / t_mm / 1e12, 1),
            "how": "1 GiB device copy (read + write); 8192^3 bf16 torch.mm"}


def append_bench(mla, A, wl, p, t, dev, stream, args):
    """mla_append_kv timed on its own (not part of the step): the step's batch
    (one new token per sequence, query rotated in place) and a bulk append of
    16 new tokens into each of 16,384 sequences (lengths U[16, 8192], one page
    per touched page slot), which is HBM-bound."""
    import numpy as np
    import torch

    def timed(fn, n):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    # the step's batch: new token at position seq_len - 1 of every sequence
    rng = np.random.default_rng(wl.seed + 77)
    c_new = torch.from_numpy(rng.standard_normal((wl.B, wl.Sq, wl.d_c), dtype=np.float32)).to(dev).bfloat16()
    r_new = torch.from_numpy(rng.standard_normal((wl.B, wl.Sq, wl.d_r), dtype=np.float32)).to(dev).bfloat16()
    q = t["q_rope"].clone()
    us_step = timed(lambda: mla.append_kv(p, c_new, r_new, t["block_table"], t["seq_lens"], t["c_kv"],
                                          t["k_pe"], t["kv_scale"], q_rope_in=q, q_rope_out=q), 20)

    # bulk: 16,384 sequences x 16 new tokens
    Bb, Sqb = 16384, 16
    lens = rng.integers(Sqb, 8192, size=Bb, endpoint=True)
    max_pages = int((lens.max() + 63) // 64)
    bt = np.full((Bb, max_pages), -1, dtype=np.int32)
    first = (lens - Sqb) // 64
    last = (lens - 1) // 64
    n_need = int((last - first + 1).sum())
    perm = rng.permutation(n_need).astype(np.int32)
    k = 0
    for b in range(Bb):
        for j in range(first[b], last[b] + 1):
            bt[b, j] = perm[k]
            k += 1
    pb = mla.make_params(Bb, Sqb, wl.H, wl.d_h, wl.d_c, wl.d_r, n_need, max_pages)
    cb = torch.empty((n_need, 64, wl.d_c), dtype=torch.bfloat16, device=dev)
    rb = torch.empty((n_need, 64, wl.d_r), dtype=torch.bfloat16, device=dev)
    cn = torch.randn((Bb, Sqb, wl.d_c), device=dev).bfloat16()
    rn = torch.randn((Bb, Sqb, wl.d_r), device=dev).bfloat16()
    btd = torch.from_numpy(bt).to(dev)
    sld = torch.from_numpy(lens.astype(np.int32)).to(dev)
    us_bulk = timed(lambda: mla.append_kv(pb, cn, rn, btd, sld, cb, rb), 20)
    nbytes = A.append_bytes(Bb * Sqb, wl.H, wl.d_c, wl.d_r)
    gbs = nbytes / (us_bulk * 1e-6) / 1e9
    return {"kernel": "mla_append_kv", "step_batch_us": round(us_step, 2),
            "step_batch_bytes": A.append_bytes(wl.B * wl.Sq, wl.H, wl.d_c, wl.d_r, with_query=True),
            "bulk": {"workload": f"{Bb} sequences x {Sqb} new tokens, lengths U[{Sqb},8192], bf16",
                     "tokens": Bb * Sqb, "us": round(us_bulk, 2), "bytes": nbytes,
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def prefill_bench(mla, A, dev, stream, args, B=4, x=4096):
    """The non-absorbed path (mla_decompress_kv + mla_prefill_attention) timed on its
    own: whole-prompt prefill of B sequences of x tokens (seq_len = x new tokens),
    DeepSeek-V3 head shapes, bf16, permuted pages, bf16 output.  Inputs are drawn
    on the device (normal(0, 1) activations, cache and RoPE keys; weights
    normal(0, 0.02)).  Each kernel's average launch duration comes from an event
    pair around each launch on its stream."""
    import numpy as np
    import torch

    H, d_h, d_c, d_r = 128, 128, 512, 64
    g = torch.Generator(device=dev)
    g.manual_seed(2024)
    pages = B * ((x + 63) // 64)
    mp = (x + 63) // 64
    perm = np.random.default_rng(2024).permutation(pages).astype(np.int32)
    bt = torch.from_numpy(perm.reshape(B, mp)).to(dev)
    sl = torch.full((B,), x, dtype=torch.int32, device=dev)

    def rnd(*shape, std=1.0):
        return (torch.randn(shape, generator=g, device=dev) * std).bfloat16()

    c_kv, k_pe = rnd(pages, 64, d_c), rnd(pages, 64, d_r)
    W_UK, W_UV = rnd(H, d_h, d_c, std=0.02), rnd(H, d_h, d_c, std=0.02)
    q_nope, q_rope = rnd(B, x, H, d_h), rnd(B, x, H, d_r)
    pp = mla.make_params(B, x, H, d_h, d_c, d_r, pages, mp, out_dtype=mla.BF16)
    L = mla.lmax(pp)
    kn = torch.empty((B, L, H, d_h), dtype=torch.bfloat16, device=dev)
    vt = torch.empty((B, H, d_h, L), dtype=torch.bfloat16, device=dev)
    out = torch.empty((B, x, H, d_h), dtype=torch.bfloat16, device=dev)

    def dec():
        mla.decompress_kv(pp, c_kv, bt, sl, W_UK, W_UV, kn, vt, stream)

    def att():
        mla.prefill_attention(pp, q_nope, q_rope, kn, vt, k_pe, bt, sl, out, stream)

    for _ in range(2):
        dec()
        att()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "non-finite prefill output"
    n = args.prefill_reps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        dec()
        ev[i][1].record(stream)
        att()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    d_us = float(np.mean([a.elapsed_time(b) for a, b, _ in ev])) * 1e3
    a_us = float(np.mean([b.elapsed_time(c) for _, b, c in ev])) * 1e3
    cost = A.prefill_cost(x, H, d_h, d_c, d_r, [x] * B, out_fmt="bf16")

    def roof(flops, us):
        t = flops / (us * 1e-6) / 1e12
        return {"us": round(us, 1), "flops": flops, "achieved": round(t, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(t / BF16_PEAK_TFLOPS, 4)}

    tot = cost.decompress_flops + cost.attention_flops
    # context for the decompression: a library GEMM of its own shape, the latent rows
    # [B*x, d_c] times [W_UK; W_UV]^T [d_c, 2*H*d_h] into one contiguous bf16 matrix
    del kn, vt
    lat = c_kv.view(-1, d_c)
    w_t = torch.cat([W_UK, W_UV]).view(2 * H * d_h, d_c).t().contiguous()
    kv_lib = torch.empty((lat.shape[0], 2 * H * d_h), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        torch.mm(lat, w_t, out=kv_lib)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(n):
        torch.mm(lat, w_t, out=kv_lib)
    g1.record(stream)
    torch.cuda.synchronize()
    lib_us = g0.elapsed_time(g1) / n * 1e3
    del kv_lib, w_t
    dec = roof(cost.decompress_flops, d_us)
    dec["library_same_shape_us"] = round(lib_us, 1)
    dec["speedup_vs_library"] = round(lib_us / d_us, 3)
    return {"workload": f"whole-prompt prefill, B={B} sequences x {x} new tokens (seq_len {x}), H={H}, "
                        f"d_h={d_h}, d_c={d_c}, d_r={d_r}, bf16, permuted pages, bf16 out",
            "tokens_per_s": round(B * x / ((d_us + a_us) * 1e-6), 0),
            "bound": "mfma",
            "decompress": dec,
            "attention": roof(cost.attention_flops, a_us),
            "path": roof(tot, d_us + a_us)}


def measured_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter summary, each counter
    scaled by its reading for a device copy of known size in the same profiling run;
    None when the summary is missing, for another workload, or was taken on a
    different version of the kernel sources."""
    try:
        kv = dict(l.split("=", 1) for l in open(COUNTERS).read().split("\n") if "=" in l and not l.startswith("#"))
        src = code_hash(KERNEL_SRCS)
    except OSError:
        return None
    if kv.get("kernel_source_sha256", "").strip() != src or kv.get("workload", "").strip() != workload:
        return None
    # each counter scaled by what it reads for a device copy of known size in the same run
    probe = float(kv["copy_probe_bytes"])
    fetch = float(kv["fetch_size_kib"]) / float(kv["copy_probe_fetch_size_kib"]) * probe
    write = float(kv["write_size_kib"]) / float(kv["copy_probe_write_size_kib"]) * probe
    return round(fetch + write)


def code_hash(paths):
    """sha256 of the sources' code: comments dropped and whitespace runs collapsed,
    so that an edit of a comment keeps the hash (string literals are kept whole)."""
    import hashlib
    import re
    tok = re.compile(r'("(?:\\.|[^"\\])*")|//[^\n]*|/\*.*?\*/', re.S)
    parts = []
    for f in paths:
        text = tok.sub(lambda m: m.group(1) or " ", open(f).read())
        parts.append(" ".join(text.split()))
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()


def cpu_baseline(case, budget_s, gpu_out):
    """The oracle, untuned, on a bounded sample: whole sequences (every head) until
    about `budget_s` seconds of CPU work; reported in the metric's unit.  Also the
    step output of the sampled rows against the GPU step's output `gpu_out`
    [B, Sq, H, d_h]: max and RMS of the error, each over the oracle output's RMS."""
    import numpy as np
    from oracle import oracle as O

    wl = case.wl
    lens = case.seq_lens.numpy()
    order = np.argsort(lens)[len(lens) // 2:]          # median-length and longer first
    t_used, toks, seqs, refs = 0.0, 0, [], []
    for b in order:
        rows = np.arange(b * wl.Sq * wl.H, (b + 1) * wl.Sq * wl.H, dtype=np.int64)
        t0 = time.perf_counter()
        out, _, _ = O.decode(case, rows=rows)
        dt = time.perf_counter() - t0
        t_used += dt
        toks += int(lens[b])
        seqs.append(int(b))
        refs.append(out)
        if t_used + dt > budget_s:
            break
    value = toks * 1152 / t_used / 1e12
    ref = np.concatenate(refs)
    got = np.concatenate([gpu_out[b].reshape(-1, wl.d_h) for b in seqs]).astype(np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = np.abs(got - ref)
    tol = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}[wl.dtype]
    parity = {"rows": int(ref.shape[0]), "sequences": seqs,
              "max_abs_err_over_rms": float(err.max() / rms), "rms_err_over_rms": float(np.sqrt(np.mean(err ** 2)) / rms),
              "tol_max_abs_over_rms": tol, "pass": bool(err.max() / rms <= tol)}
    return ({"value": value, "unit": "TB/s", "cores": O.num_threads(), "kind": "oracle",
             "sample": f"{len(seqs)} whole sequences ({toks} tokens, all {wl.H} heads) of the "
                       f"same workload, fp64 oracle, {t_used:.1f} s"}, parity)


if __name__ == "__main__":
    main()
