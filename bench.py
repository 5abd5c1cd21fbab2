#!/usr/bin/env python3
"""Throughput of one rank's decode-attention share over a paged latent KV head
on one MI355X, through libsplash_attn's C ABI.

Default workload: the transition batch, the largest single-GPU case: 64
requests with context lengths drawn log-uniform in [512, 65,536] (856,942 KV
tokens), 128 query heads sharing one latent KV row of 576 bf16 dims (V = the
first 512), page size 64, randomly permuted pages, each request owned whole
(the DP-attention / DOP owner share).
One step = one pass of the whole hot path over one batch:
  * splash_decode_attn over the batch (split-KV chunks + their merge), and
  * splash_kv_repack of a seeded half of the batch's requests (all their
    pages) to a freshly permuted destination pool (the handoff copy).
Inputs are resident in HBM before timing starts; the timed steps rotate over
several copies of the inputs (more bytes than the 256 MiB Infinity Cache) so
that KV reads come from HBM.

Prints ONE JSON line: KV tokens/s over the step, the decode kernel's HBM
roofline (algorithmic bytes / its measured duration), and the CPU oracle's
throughput on a bounded sample of the same workload.

Pages cited: the weekinpapers page is "SPLASH: Switching Parallel Layouts of Attention with
Seamless Handoff for LLM Serving" (weekinpapers.com); the thelatestinai page is that paper's
summary with its appendix tables (thelatestinai.com).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
KV_ROW_BYTES = 576 * 2


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="transition",
                    help="owner | tp | cp | transition | sweep:<owner|tp|cp|gqa<G>>:<ctx>")
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-repack", action="store_true", help="time decode attention alone")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured-peak runs (MFMA loop, streaming read) after the timed steps")
    ap.add_argument("--layout-model", action="store_true",
                    help="instead of the throughput line: time the busiest rank's attention share of each layout "
                         "(B=16, T=8, H=128, contexts 1k..64k) and pick the cheapest layout per context")
    ap.add_argument("--handoff", type=int, default=0, metavar="K",
                    help="instead of the throughput line: spread the repack of a seeded half of the requests over "
                         "K decode steps on a second stream and report the decode-step slowdown")
    return ap.parse_args()


def build_workload(name):
    import workloads as W
    repack = False
    merge = None
    splits = 0
    if name == "owner":
        case, repack = W.case_owner(), True
        desc = "request-owned share (DP-attention/DOP owner): B=16 x 4,096 tokens, 128 heads, 576/512 bf16, page 64"
    elif name == "tp":
        case, splits = W.case_tp(), 8
        desc = "head-sliced share (TP rank): B=16 x 16,384 tokens, heads [0,16) of 128, 8 split-KV chunks + merge"
    elif name == "cp":
        case, merge = W.case_cp(), W.case_cp_merge()
        desc = "token-split share (CP rank 3/8): B=16 x 65,536, tokens [24,576, 32,768), 128 heads; merge of 8 sets"
    elif name == "transition":
        case, repack = W.case_transition(), True
        desc = "transition batch: 64 requests log-uniform [512, 65,536], 128 heads; repack of 32 requests"
    elif name.startswith("sweep:"):
        _, share, ctx = name.split(":")
        case = W.sweep_case(share, int(ctx))
        desc = f"sweep: {share} share, B=16 x {ctx} tokens"
    else:
        raise SystemExit(f"unknown workload {name}")
    return case, desc, repack, merge, splits


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of a layout; --gpus {args.gpus} is not supported: "
              "the library runs on a single MI355X (the multi-GPU exchange of a layout is not implemented).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import layout_agnostic_latent_amd as sp
    import workloads as W

    dev = torch.device("cuda:0")
    if args.layout_model:
        return run_layout_model(args)
    case, desc, do_repack, merge_case, splits = build_workload(args.workload)
    if args.handoff > 0:
        return run_handoff(args, case, desc, splits)
    if args.no_repack:
        do_repack = False
    B, Hs = case.num_reqs, case.num_q_heads
    kv_tokens = case.kv_tokens()
    pool_bytes = case.kv_pages.nbytes
    copies = args.copies or max(2, min(8, math.ceil(1.2e9 / pool_bytes)))

    # ---- inputs, resident in HBM ----
    q0 = torch.from_numpy(case.q.view(np.int16)).to(dev)
    kv0 = torch.from_numpy(case.kv_pages.view(np.int16)).to(dev)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.seq_lens).to(dev)
    qs = [q0] + [q0.clone() for _ in range(copies - 1)]
    kvs = [kv0] + [kv0.clone() for _ in range(copies - 1)]
    out = torch.empty((B, Hs, case.d_v), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hs), dtype=torch.float32, device=dev)
    rep = None
    if do_repack:
        rc = W.make_repack_case(case, seed=case.seed + 100)
        rep = dict(st=torch.from_numpy(rc.src_table).to(dev), dt=torch.from_numpy(rc.dst_table).to(dev),
                   dst=[torch.empty((rc.dst_num_pages,) + case.kv_pages.shape[1:], dtype=torch.int16, device=dev)
                        for _ in range(copies)],
                   pages=rc.dst_num_pages)
    mrg = None
    if merge_case is not None:
        mrg = dict(P=torch.from_numpy(merge_case.partials).to(dev), L=torch.from_numpy(merge_case.lses).to(dev))
        mrg["out"] = torch.empty(mrg["P"].shape[1:], dtype=torch.float32, device=dev)
        mrg["lse"] = torch.empty(mrg["P"].shape[1:2], dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(i):
        k = i % copies
        sp.decode_attn(qs[k], kvs[k], bt, sl, case.head_lo, case.head_hi, case.tok_lo, case.tok_hi, out, lse,
                       d_v=case.d_v, scale=case.scale, num_splits=splits)
        if mrg is not None:
            sp.lse_merge(mrg["P"], mrg["L"], mrg["out"], mrg["lse"])
        if rep is not None:
            sp.kv_repack(kvs[k], rep["st"], rep["dst"][k], rep["dt"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region 1: the step, nothing else on the stream ----
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # ---- timed region 2: the same steps, each kernel bracketed by HIP events ----
    sp.profile_start()
    for i in range(args.steps):
        step(i)
    prof = sp.profile_stop()
    assert sp.device_errors(clear=True) == 0

    dec_n = prof["decode_launches"]
    dec_us = 1e3 * prof["decode_ms"] / max(1, dec_n)
    n_split_merges = dec_n if sp.decode_plan(B, case.num_heads, case.d_qk, case.d_v, case.page_size,
                                             case.max_pages_per_req, case.num_pages, case.scale, case.head_lo,
                                             case.head_hi, case.tok_lo, case.tok_hi, splits)[0] > 1 else 0
    merge_us = 1e3 * prof["merge_ms"] / max(1, prof["merge_launches"])
    lse_merge_us = 1e3 * prof["lse_merge_ms"] / max(1, prof["lse_merge_launches"])
    repack_us = 1e3 * prof["repack_ms"] / max(1, prof["repack_launches"])

    # algorithmic bytes and flops of one decode-attention call
    dec_bytes = (kv_tokens * KV_ROW_BYTES * case.num_kv_heads + B * Hs * case.d_qk * 2 + B * Hs * case.d_v * 4
                 + B * Hs * 4
                 + case.block_table.nbytes + case.seq_lens.nbytes)
    dec_flops = 2.0 * Hs * (case.d_qk + case.d_v) * kv_tokens
    achieved = dec_bytes / (dec_us * 1e-6) / 1e9
    call_us = dec_us + (merge_us if n_split_merges else 0.0)

    parts = {
        "decode_kernel_us": round(dec_us, 2),
        "split_merge_kernel_us": round(merge_us, 2) if n_split_merges else None,
        "decode_call_us": round(call_us, 2),
        "decode_call_GBps": round(dec_bytes / (call_us * 1e-6) / 1e9, 1),
        "decode_TFLOPs": round(dec_flops / (dec_us * 1e-6) / 1e12, 1),
        "decode_mfma_frac": round(dec_flops / (dec_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "decode_kv_tokens_per_s": round(kv_tokens / (dec_us * 1e-6), 1),
        "algorithmic_bytes_per_decode": int(dec_bytes),
    }
    if rep is not None:
        moved = rep["pages"] * case.kv_pages[0].nbytes
        parts["repack_kernel_us"] = round(repack_us, 2)
        parts["repack_bytes_moved"] = int(moved)
        parts["repack_TBps_rw"] = round(2 * moved / (repack_us * 1e-6) / 1e12, 3)
        parts["repack_hbm_frac"] = round(2 * moved / (repack_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    if mrg is not None:
        mb = mrg["P"].numel() * 4 + mrg["L"].numel() * 4 + mrg["out"].numel() * 4 + mrg["lse"].numel() * 4
        parts["lse_merge_us"] = round(lse_merge_us, 2)
        parts["lse_merge_TBps"] = round(mb / (lse_merge_us * 1e-6) / 1e12, 3)

    traffic = measured_traffic(args.workload, "decode_attn")

    # Peaks of this GPU as measured (after the timed regions): the fractions
    # above use the published peaks; these say what the chip sustains.
    peaks = None
    if not args.no_peaks:
        buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        buf.fill_(1)
        pk = sp.measure_peaks(buf)
        copy_gbps = device_copy_rate(buf)
        del buf
        dec_tflops = dec_flops / (dec_us * 1e-6) / 1e12
        peaks = {"mfma_bf16_TFLOPs": round(pk["mfma_bf16_tflops"], 1),
                 "mfma_clock_GHz": round(pk["mfma_clock_ghz"], 3),
                 "hbm_read_GBps": round(pk["hbm_read_gbps"], 1),
                 "copy_rw_GBps": round(copy_gbps, 1),
                 "decode_frac_of_measured_read": round(achieved / pk["hbm_read_gbps"], 4),
                 "decode_frac_of_measured_mfma": round(dec_tflops / pk["mfma_bf16_tflops"], 4),
                 "how": "splash_measure_peaks: v_mfma_f32_32x32x16_bf16 loop on every SIMD (~2 ms, best of 3), "
                        "shader clock from s_memtime / s_memrealtime; non-temporal streaming read of 1 GiB; "
                        "copy_rw_GBps: torch's device-to-device copy of 512 MiB (read + write bytes), best of 5"}
        if rep is not None:
            peaks["repack_frac_of_measured_copy"] = round(parts["repack_TBps_rw"] * 1e3 / copy_gbps, 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, args.cpu_seconds)

    line = {
        "metric": "decode-attn KV tokens/s + % of HBM/MFMA roofline, 128-head latent KV, 1 GPU",
        "value": round(kv_tokens / (ms_per_step * 1e-3), 1),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "num_reqs": B, "kv_tokens": kv_tokens, "heads": Hs, "d_qk": case.d_qk,
                   "d_v": case.d_v, "page_size": case.page_size, "input_copies": copies,
                   "step": "decode_attn" + (" + lse_merge" if mrg is not None else "")
                           + (" + kv_repack(half of the requests)" if rep is not None else "")},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_attn16_kernel" if case.d_qk == 576 and min(Hs, case.q.shape[1]
                                                                                   // case.num_kv_heads) <= 16
                     else "decode_attn_kernel"},
        "parts": parts,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        "library": sp.library_info(),
    }
    print(json.dumps(line), flush=True)


def run_handoff(args, case, desc, splits):
    """Background handoff on one GPU: the pages of a seeded half of the
    requests move to a fresh pool in K slices (one per decode step) on a
    second stream of default priority, while decode attention over the batch
    runs on the first; both read the same KV pool.  Reports how much longer a
    decode step takes while the handoff runs (the pages' switch cost: a
    median below 0.51% of the step, weekinpapers page, Abstract)."""
    import numpy as np
    import torch

    import layout_agnostic_latent_amd as sp
    import workloads as W

    dev = torch.device("cuda:0")
    K = args.handoff
    B, Hs = case.num_reqs, case.num_q_heads
    q = torch.from_numpy(case.q.view(np.int16)).to(dev)
    kv = torch.from_numpy(case.kv_pages.view(np.int16)).to(dev)
    bt = torch.from_numpy(case.block_table).to(dev)
    sl = torch.from_numpy(case.seq_lens).to(dev)
    out = torch.empty((B, Hs, case.d_v), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hs), dtype=torch.float32, device=dev)
    rc = W.make_repack_case(case, seed=case.seed + 100)
    dst = torch.zeros((rc.dst_num_pages,) + case.kv_pages.shape[1:], dtype=torch.int16, device=dev)
    rows = np.array_split(np.arange(rc.src_table.shape[0]), K)
    slices = [(torch.from_numpy(np.ascontiguousarray(rc.src_table[r])).to(dev),
               torch.from_numpy(np.ascontiguousarray(rc.dst_table[r])).to(dev)) for r in rows if len(r)]
    errs = torch.zeros((1,), dtype=torch.int32, device=dev)
    side = torch.cuda.Stream(device=dev)  # default priority
    main = torch.cuda.current_stream(dev)

    def decode():
        sp.decode_attn(q, kv, bt, sl, case.head_lo, case.head_hi, case.tok_lo, case.tok_hi, out, lse,
                       d_v=case.d_v, scale=case.scale, num_splits=splits, stream=main)

    def repack(i):
        st, dt = slices[i % len(slices)]
        sp.kv_repack(kv, st, dst, dt, errs, stream=side)

    def timed(fn, n, streams):
        starts = {s_: torch.cuda.Event(enable_timing=True) for s_ in streams}
        ends = {s_: torch.cuda.Event(enable_timing=True) for s_ in streams}
        torch.cuda.synchronize()
        for s_ in streams:
            starts[s_].record(s_)
        for i in range(n):
            fn(i)
        for s_ in streams:
            ends[s_].record(s_)
        torch.cuda.synchronize()
        t0 = min(starts.values(), key=lambda e: 0)  # all recorded back to back
        return {s_: t0.elapsed_time(ends[s_]) for s_ in streams}

    for _ in range(args.warmup):
        decode()
        repack(0)
    torch.cuda.synchronize()
    # K decode steps alone, then K steps with one handoff slice each, in
    # rounds; medians over the rounds
    n = len(slices)
    rounds = max(3, min(9, args.steps // max(1, n)))
    a_s, b_s, r_s, d_s = [], [], [], []
    for _ in range(rounds):
        a_s.append(timed(lambda i: decode(), n, [main])[main] / n)
        both = timed(lambda i: (decode(), repack(i)), n, [main, side])
        b_s.append(both[main] / n)
        d_s.append(both[side])
        r_s.append(timed(lambda i: repack(i), n, [side])[side])
    alone, step_both = float(np.median(a_s)), float(np.median(b_s))
    rep_alone, done_after = float(np.median(r_s)), float(np.median(d_s))
    assert int(errs.item()) == 0 and sp.device_errors(clear=True) == 0
    moved = rc.dst_num_pages * case.kv_pages[0].nbytes
    # the handoff really happened: every moved page equals its source
    src_idx = torch.from_numpy(rc.src_table[rc.src_table >= 0]).long().to(dev)
    dst_idx = torch.from_numpy(rc.dst_table[rc.dst_table >= 0]).long().to(dev)
    assert torch.equal(dst[dst_idx], kv[src_idx]), "handoff copy differs from its source"
    line = {
        "metric": "decode-step slowdown while a background KV handoff runs on a second stream, 1 GPU",
        "value": round(100.0 * (step_both / alone - 1.0), 3),
        "unit": "% of the decode step",
        "higher_is_better": False,
        "n_gpus": 1,
        "steps": n * rounds,
        "warmup": args.warmup,
        "data": "synthetic",
        "config": {"workload": desc, "handoff_slices": n, "moved_pages": int(rc.dst_num_pages),
                   "moved_bytes": int(moved),
                   "streams": "decode on the current stream, repack on a second stream, both default priority"},
        "parts": {"decode_step_alone_us": round(alone * 1e3, 2), "decode_step_during_handoff_us": round(step_both * 1e3, 2),
                  "repack_alone_us": round(rep_alone * 1e3, 2),
                  "repack_alone_TBps_rw": round(2 * moved / (rep_alone * 1e-3) / 1e12, 3),
                  "handoff_done_after_us": round(done_after * 1e3, 2), "rounds": rounds},
    }
    print(json.dumps(line))


def run_layout_model(args, B=16, T=8, H=128, contexts=(1024, 4096, 16384, 32768, 65536)):
    """Attention time per decode step of each layout, as the busiest rank's
    share time measured at its real shape (layout_model's decomposition of
    thelatestinai page, Appendix Table 2), and the cheapest layout."""
    import numpy as np
    import torch

    import layout_agnostic_latent_amd as sp
    import workloads as W
    from layout_agnostic_latent_amd import layout_model as lm

    dev = torch.device("cuda:0")

    def time_share(sh, s):
        # a rank's share: sh.reqs requests, sh.tokens tokens each (for CP the
        # range of rank 3 of a history of s tokens), sh.heads query heads
        if sh.reqs == 0 or sh.tokens == 0:
            return 0.0
        cp = sh.merge_parts > 1
        lo = 3 * s // T if cp else 0
        hi = lo + sh.tokens if cp else s
        case = W.make_decode_case("share", 7, [s] * sh.reqs, num_heads=H, d_qk=W.LATENT_QK, d_v=W.LATENT_V,
                                  page_size=64, scale=W.LATENT_SCALE, head_lo=0, head_hi=sh.heads,
                                  tok_lo=lo, tok_hi=hi, live_only_in_range=cp)
        copies = max(2, min(16, math.ceil(6e8 / case.kv_pages.nbytes)))
        qs = [torch.from_numpy(case.q.view(np.int16)).to(dev) for _ in range(copies)]
        kvs = [torch.from_numpy(case.kv_pages.view(np.int16)).to(dev) for _ in range(copies)]
        bt = torch.from_numpy(case.block_table).to(dev)
        sl = torch.from_numpy(case.seq_lens).to(dev)
        out = torch.empty((sh.reqs, sh.heads, case.d_v), dtype=torch.float32, device=dev)
        lse = torch.empty((sh.reqs, sh.heads), dtype=torch.float32, device=dev)
        # CP: after a reduce-scatter by head, each rank merges T parts of its H/T heads
        mh = max(1, H // T)
        parts = torch.randn((T, sh.reqs * mh, case.d_v), dtype=torch.float32, device=dev)
        plse = torch.rand((T, sh.reqs * mh), dtype=torch.float32, device=dev) * 10 - 5
        mout = torch.empty((sh.reqs * mh, case.d_v), dtype=torch.float32, device=dev)
        mlse = torch.empty((sh.reqs * mh,), dtype=torch.float32, device=dev)

        def call(i):
            k = i % copies
            sp.decode_attn(qs[k], kvs[k], bt, sl, 0, sh.heads, lo, hi, out, lse, d_v=case.d_v, scale=case.scale)
            if cp:
                sp.lse_merge(parts, plse, mout, mlse)

        for i in range(3):
            call(i)
        n = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        del qs, kvs
        torch.cuda.empty_cache()
        return e0.elapsed_time(e1) / n * 1e3  # us

    rows = []
    for s in contexts:
        cache = {}

        def time_of(sh, s=s, cache=cache):
            if sh not in cache:
                cache[sh] = time_share(sh, s)
            return cache[sh]

        best, times = lm.choose(B, T, s, H, time_of)
        rows.append({"context": s, "attention_us": {k: round(v, 2) for k, v in times.items()}, "best": best})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    line = {
        "metric": "attention time per decode step of each layout (busiest rank's measured share), 1 GPU",
        "unit": "us",
        "higher_is_better": False,
        "n_gpus": 1,
        "data": "synthetic",
        "config": {"workload": f"B={B} requests, T={T} ranks, H={H} query heads, one 576-dim latent KV head, page 64",
                   "shares": "TP: H/T heads of every request; CP: 1/T of every request's tokens + merge of T parts "
                             "over H/T heads; DP-attention/DOP: ceil(B/T) whole requests"},
        "rows": rows,
    }
    print(json.dumps(line))


def device_copy_rate(buf):
    """Read + write GB/s of torch's device-to-device copy between the two
    halves of `buf` (best of 5), the box's own copy rate next to the 8 TB/s
    published peak."""
    import torch
    half = buf.numel() // 2
    a, b = buf[:half], buf[half:2 * half]
    b.copy_(a)
    best = float("inf")
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    return 2 * half / (best * 1e-3) / 1e9


def measured_traffic(workload, kernel_prefix):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary of this workload (profiles/decode_attn_<workload>.json),
    or None if there is none or the kernel source changed since it was taken."""
    from layout_agnostic_latent_amd.rocprof_summary import kernel_source_hash
    path = os.path.join(ROOT, "profiles", f"decode_attn_{workload.replace(':', '_')}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    for k, r in rec.get("kernels", {}).items():
        if k.startswith(kernel_prefix) and "traffic_bytes" in r:
            return r["traffic_bytes"]
    return None


def cpu_baseline(case, budget_s):
    """The float64 oracle on the host cores, on requests of the same batch, for about budget_s seconds; then
    the same with BLAS limited to one thread, for a third of that."""
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0))
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max([p.get("num_threads", 1) for p in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:  # pragma: no cover
        threads, threadpool_limits = cores, None

    def run(seconds):
        done_tokens = 0
        reqs = 0
        t0 = time.perf_counter()
        b = 0
        while True:
            oracle.decode_attn(case.q, case.kv_pages, case.block_table, case.seq_lens, case.head_lo, case.head_hi,
                               case.tok_lo, case.tok_hi, case.d_v, case.page_size, case.scale, reqs=[b])
            lo = max(case.tok_lo, 0)
            done_tokens += max(0, min(case.tok_hi, int(case.seq_lens[b])) - lo)
            reqs += 1
            b = (b + 1) % case.num_reqs
            el = time.perf_counter() - t0
            if el >= seconds:
                return done_tokens, reqs, el

    done_tokens, reqs, el = run(budget_s)
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            t1, _, e1 = run(budget_s / 3.0)
        one = round(t1 / e1, 1)
    return {"value": round(done_tokens / el, 1), "unit": "KV tokens/s", "cores": int(threads), "kind": "oracle",
            "value_1_thread": one, "blas": blas,
            "sample": f"{reqs} requests of the same batch (float64 numpy, {done_tokens} KV tokens, {el:.1f} s; "
                      f"{cores} cores in the affinity mask); value_1_thread: the same loop with BLAS limited to one "
                      f"thread for {budget_s / 3.0:.1f} s"}


if __name__ == "__main__":
    main()
