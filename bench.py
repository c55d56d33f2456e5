#!/usr/bin/env python3
"""Benchmark of the paged KV-cache attention forward pass on one MI355X.

One step = one whole forward call of the MHA decode workload (32 q = 32 kv
heads x 128, fp16, page size 16): the new token of every sequence is appended
into its page, then every sequence attends over its cache (context 4096 + the
new token), batch 256.  Inputs are seeded synthetic data resident in HBM
before timing starts.  `value` is the whole-job decode rate in GB/s of
algorithmic bytes (the K/V rows the method must read, q, out, lse, the table
entries and metadata, plus the appended rows read and written).

Printed as ONE JSON line, with
  roofline     the attention kernel alone: algorithmic bytes per launch over
               its mean launch time (HIP events on the launch stream), against
               the 8 TB/s HBM peak;
  cpu_baseline the CPU fp64 oracle timed on the host on a bounded sample of
               the same workload (whole sequences), scaled to GB/s;
  prefill      the causal-prefill-with-append workload (batch 4 x 2048 new
               tokens, 32 x 128, fp16, empty cache) in TFLOP/s of causal
               attention flops against the 2.5 PFLOP/s dense fp16 MFMA peak.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFS = 2500.0
METRIC = "paged-attn decode HBM GB/s + prefill TFLOP/s, as fraction of MI355X peak"


def algorithmic_bytes(case, elt=2):
    """Bytes the method must move for one call (visible K/V, q, out, lse,
    table entries, metadata; plus append traffic)."""
    Kb = case.keys_visible()
    hkv, hq, d = case.num_heads_kv, case.num_heads_q, case.head_dim
    T = case.total_q
    P = case.page_size or 1
    b = sum(Kb) * hkv * d * 2 * elt
    b += T * hq * d * elt * 2 + T * hq * 4
    if case.page_size:
        b += sum(-(-k // P) for k in Kb) * 4
    b += (2 * case.batch + 1) * 4
    if case.append:
        b += 2 * T * hkv * d * elt * 2
    return b


def causal_flops(case):
    """4 * D * Hq * sum over query rows of the keys each row can see."""
    total = 0
    for L, n in zip(case.cache_seqlens, case.q_lens):
        K = L + (n if case.append else 0)
        if case.causal:
            # rows i = 0..n-1 see K - n + i + 1 keys
            total += n * (K - n) + n * (n + 1) // 2
        else:
            total += n * K
    return 4 * case.head_dim * case.num_heads_q * total


# every source the decode kernel is built from (the prefill unit is not part of it)
KERNEL_SOURCES = ("paged_kv_cache_lds_amd/csrc/pa_device.h", "paged_kv_cache_lds_amd/csrc/pa_common.h",
                  "paged_kv_cache_lds_amd/csrc/pa_decode.h", "paged_kv_cache_lds_amd/csrc/pa_kernels.h",
                  "paged_kv_cache_lds_amd/csrc/paged_attn.hip")
TRAFFIC_PROFILE = "profiles/attn_decode_mha_decode_b256_ctx4096.txt"


def measured_traffic(batch, ctx):
    """HBM bytes per attention launch measured with rocprofv3 PMC counters
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated) on the default workload, taken
    from the committed profile summary -- or None if the workload differs or
    the kernel sources changed since the counters were taken."""
    import hashlib
    if (batch, ctx) != (256, 4096):
        return None
    try:
        text = open(os.path.join(ROOT, TRAFFIC_PROFILE)).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines()
                  if line.startswith(("kernel_source_sha256:", "traffic_bytes_per_launch:")))
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if fields.get("kernel_source_sha256", "").strip() != h.hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"].strip())


def time_calls(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps     # ms per call


def median_call_ms(fn, reps, torch, flush=None):
    """Median time of single calls, each bracketed by events on the current
    stream, with `flush` (a 1 GiB HBM read that evicts L2 and the 256 MiB
    Infinity Cache) run between calls outside the timed region."""
    times = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    times.sort()
    return times[len(times) // 2], times[0]


def sweep(name, reps, out_path):
    """Measurement sweeps over the workload families (one JSON object per
    point, appended to `out_path`); each point reports median / min call time
    and the fraction of its roofline."""
    import numpy as np
    import torch

    import paged_kv_cache_lds_amd as pa
    import workloads as wl

    torch.cuda.set_device(0)
    # cache flush between timed calls: stream-read 1 GiB (evicts L2 and the
    # 256 MiB Infinity Cache with clean lines, so no write-back lands in the
    # next timed call)
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush = lambda: scratch.sum()
    fh = open(out_path, "a")

    def emit(rec):
        fh.write(json.dumps(rec) + "\n")
        fh.flush()
        print(json.dumps(rec), file=sys.stderr, flush=True)

    def make_call(case, inp, num_splits=None, max_seqlen_k=None, seqlens=None, append=None,
                  rot=None, aux=None):
        kn = inp.k_new if (append if append is not None else case.append) else None
        vn = inp.v_new if kn is not None else None
        seq = inp.cache_seqlens if seqlens is None else seqlens
        out = torch.empty_like(inp.q)
        lse = torch.empty(inp.q.shape[:2], dtype=torch.float32, device="cuda")
        args = pa.make_args(inp.q, inp.k_cache, inp.v_cache, inp.block_table, seq,
                            inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q,
                            max_seqlen_k=max_seqlen_k if max_seqlen_k is not None else inp.max_seqlen_k,
                            k_new=kn, v_new=vn, causal=case.causal,
                            num_splits=case.num_splits if num_splits is None else num_splits,
                            out=out, softmax_lse=lse)
        S = pa.paged_attn_splits_for(args)
        ws = torch.empty(max(1, pa.paged_attn_workspace_size(args)), dtype=torch.uint8, device="cuda")
        rk = {} if rot is None else dict(rotary_cos=rot[0], rotary_sin=rot[1],
                                         rotary_interleaved=rot[2])

        def call():
            pa.paged_attn_fwd(inp.q, inp.k_cache, inp.v_cache, inp.block_table, seq,
                              inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q,
                              max_seqlen_k=args.max_seqlen_k, k_new=kn, v_new=vn,
                              causal=case.causal, num_splits=args.num_splits, out=out,
                              softmax_lse=lse, workspace=ws, aux_stream=aux, **rk)
        return S, call

    def run(case, inp, **kw):
        S, call = make_call(case, inp, **kw)
        call()
        torch.cuda.synchronize()
        med, mn = median_call_ms(call, reps, torch, flush)
        return S, med, mn

    if name == "copy":
        n = 1 << 31   # 4 GiB of fp16 read + written
        a = torch.empty(n, dtype=torch.float16, device="cuda")
        b = torch.empty_like(a)
        med, mn = median_call_ms(lambda: b.copy_(a), reps, torch, flush)
        emit({"sweep": "copy", "bytes": 4 * n, "ms": med, "GBps": 4 * n / med / 1e6})
    elif name == "decode":
        # MHA decode, 32 x 128 fp16: one pool per page size reused for every
        # (batch, context) point through the leading table rows
        for P in (16, 256):
            big = wl.mha_decode(256, 4096, page_size=P)
            inp = wl.make_inputs(big, "cuda")
            for ctx in (512, 1024, 2048, 4096):
                for B in (1, 2, 4, 8, 16, 32, 64, 128, 256):
                    c = wl.mha_decode(B, ctx, page_size=P)
                    c.causal = False
                    sub = wl.Inputs(case=c, q=inp.q[:B].contiguous(), k_cache=inp.k_cache,
                                    v_cache=inp.v_cache,
                                    block_table=inp.block_table[:B].contiguous(),
                                    cache_seqlens=torch.full((B,), ctx, dtype=torch.int32,
                                                             device="cuda"),
                                    cu_seqlens_q=inp.cu_seqlens_q[:B + 1].contiguous(),
                                    k_new=None, v_new=None, max_seqlen_q=1, max_seqlen_k=ctx,
                                    pages_of=[])
                    S, med, mn = run(c, sub)
                    by = algorithmic_bytes(c)
                    rec = {"sweep": "decode", "P": P, "batch": B, "ctx": ctx, "splits": S,
                           "ms": med, "ms_min": mn, "GBps": by / med / 1e6,
                           "frac": by / med / 1e6 / HBM_PEAK_GBS}
                    if P == 16:
                        # forced split budgets beside the heuristic's
                        forced = {}
                        for fs in (1, 2, 4, 8):
                            forced[fs] = med if fs == S else run(c, sub, num_splits=fs)[1]
                        best = min(forced, key=forced.get)
                        rec.update({"forced_ms": forced, "best_splits": best,
                                    "heuristic_over_best": med / min(med, forced[best])})
                    emit(rec)
            del inp
            torch.cuda.empty_cache()
    elif name == "gqa":
        for paged in (True, False):
            c = wl.gqa_long_split(paged=paged)
            inp = wl.make_inputs(c, "cuda")
            by = algorithmic_bytes(c)
            for hint in ("alloc", "max"):
                mk = 131072 if hint == "alloc" else max(c.cache_seqlens)
                S, med, mn = run(c, inp, num_splits=0, max_seqlen_k=mk)
                emit({"sweep": "gqa", "paged": paged, "splits": S, "heuristic": hint,
                      "ms": med, "ms_min": mn, "GBps": by / med / 1e6,
                      "frac": by / med / 1e6 / HBM_PEAK_GBS})
            for s in (1, 2, 4, 8, 16, 32, 64, 128):
                S, med, mn = run(c, inp, num_splits=s)
                emit({"sweep": "gqa", "paged": paged, "splits": S, "heuristic": None,
                      "ms": med, "ms_min": mn, "GBps": by / med / 1e6,
                      "frac": by / med / 1e6 / HBM_PEAK_GBS})
            del inp
            torch.cuda.empty_cache()
        # the same heads and allocation with short live lengths (64..512): the
        # host sizes the budget from the allocation, the device caps splits
        # at >= 8 key tiles each
        rng = np.random.default_rng(2500)
        lens = [int(x) for x in rng.integers(64, 512, size=8, endpoint=True)]
        c = wl.Case(**{**wl.gqa_long_split(True).__dict__, "name": "gqa_short_in_long_alloc",
                       "cache_seqlens": lens, "seed": 2500})
        inp = wl.make_inputs(c, "cuda")
        by = algorithmic_bytes(c)
        for s in (0, 1, 8, 32, 128):
            S, med, mn = run(c, inp, num_splits=s)
            emit({"sweep": "gqa", "paged": True, "lengths": "64..512", "splits": S,
                  "heuristic": "alloc" if s == 0 else None, "ms": med, "ms_min": mn,
                  "GBps": by / med / 1e6, "frac": by / med / 1e6 / HBM_PEAK_GBS})
        del inp
        torch.cuda.empty_cache()
    elif name == "prefill":
        for nq, prefix in ((170, "zero"), (170, "uniform"), (2048, "zero"), (2048, "uniform"),
                           (8192, "zero")):
            c = wl.causal_prefill_append(nq, prefix)
            inp = wl.make_inputs(c, "cuda")
            S, med, mn = run(c, inp)
            # attention alone on the same keys (the rows are in the pages by now)
            seq_after = inp.cache_seqlens + c.q_lens[0]
            _, amed, _ = run(c, inp, seqlens=seq_after, append=False)
            fl = causal_flops(c)
            emit({"sweep": "prefill", "nq": nq, "prefix": prefix, "ms": med, "ms_min": mn,
                  "TFLOPs": fl / med / 1e9, "frac": fl / med / 1e9 / MFMA_F16_PEAK_TFS,
                  "attention_only_ms": amed,
                  "attention_only_frac": fl / amed / 1e9 / MFMA_F16_PEAK_TFS})
            del inp
            torch.cuda.empty_cache()
    elif name == "unified":
        for heads, hd in ((32, 128), (12, 64)):
            for nq in (100, 500, 1000):
                c = wl.unified_varlen(nq, heads=heads, head_dim=hd)
                inp = wl.make_inputs(c, "cuda")
                S, med, mn = run(c, inp)
                # the other plans of a mixed batch: the two launches concurrent
                # on two streams, and one unified launch
                _, cmed, _ = run(c, inp, aux="auto")
                os.environ["PAGED_ATTN_SINGLE_KERNEL"] = "1"
                _, smed, _ = run(c, inp)
                del os.environ["PAGED_ATTN_SINGLE_KERNEL"]
                by, fl = algorithmic_bytes(c), causal_flops(c)
                t_roof = max(by / (HBM_PEAK_GBS * 1e9), fl / (MFMA_F16_PEAK_TFS * 1e12)) * 1e3
                # the same work as two calls: decode rows, then the prefill chunk
                dec = wl.Case(**{**c.__dict__, "q_lens": c.q_lens[1:],
                                 "cache_seqlens": c.cache_seqlens[1:]})
                pre = wl.Case(**{**c.__dict__, "q_lens": c.q_lens[:1],
                                 "cache_seqlens": c.cache_seqlens[:1]})
                di = wl.make_inputs(dec, "cuda")
                pi = wl.make_inputs(pre, "cuda")
                _, dmed, _ = run(dec, di)
                _, pmed, _ = run(pre, pi)
                dby = algorithmic_bytes(dec)
                emit({"sweep": "unified", "nq": nq, "heads": heads, "head_dim": hd, "splits": S,
                      "ms": med, "ms_min": mn, "roofline_ms": t_roof, "frac": t_roof / med,
                      "concurrent_ms": cmed, "one_launch_ms": smed, "two_call_ms": dmed + pmed,
                      "decode_only_ms": dmed,
                      "decode_only_frac": dby / (HBM_PEAK_GBS * 1e9) * 1e3 / dmed})
                del inp, di, pi
                torch.cuda.empty_cache()
    elif name == "plan":
        # the plan's unit shape and split budget on all-decode batches whose
        # unit counts fall between whole multiples of the compute units,
        # beside forced alternatives: one-head or pair units
        # (PAGED_ATTN_HEAD_PAIRS=0 / 2), one or two splits; every sequence at
        # `ctx` cached keys, no append
        points = [(32, 32, 128, B, 4096) for B in (12, 20, 24, 40, 48, 50, 60, 96, 100)]
        points += [(32, 32, 128, 12, 2048), (32, 32, 128, 20, 8192), (32, 32, 128, 52, 2048),
                   (32, 8, 128, 48, 8192), (32, 8, 128, 200, 4096),
                   (12, 12, 64, 96, 4096), (12, 12, 64, 128, 4096), (12, 12, 64, 200, 2048),
                   (32, 32, 64, 128, 4096)]
        env0 = os.environ.get("PAGED_ATTN_HEAD_PAIRS")
        for hq, hkv, hd, B, ctx in points:
            c = wl.Case(name=f"plan_{hq}x{hkv}x{hd}_b{B}_ctx{ctx}", q_lens=[1] * B,
                        cache_seqlens=[ctx] * B, num_heads_q=hq, num_heads_kv=hkv, head_dim=hd,
                        dtype="f16", page_size=16, append=False, causal=False,
                        seed=6000 + B + ctx + hkv + hd)
            inp = wl.make_inputs(c, "cuda")
            by = algorithmic_bytes(c)
            rec = {"sweep": "plan", "heads": f"{hq}/{hkv}", "head_dim": hd, "batch": B, "ctx": ctx,
                   "units_one_head": B * hkv}
            for label, pm, ns in (("plan", None, 0), ("one_S1", "0", 1), ("one_S2", "0", 2),
                                  ("pairs_S1", "2", 1), ("pairs_S2", "2", 2)):
                if pm is None:
                    os.environ.pop("PAGED_ATTN_HEAD_PAIRS", None)
                else:
                    os.environ["PAGED_ATTN_HEAD_PAIRS"] = pm
                S, med, mn = run(c, inp, num_splits=ns)
                rec[label + "_ms"] = med
                if label == "plan":
                    rec.update({"plan_splits": S, "plan_GBps": by / med / 1e6,
                                "plan_frac": by / med / 1e6 / HBM_PEAK_GBS})
            if env0 is None:
                os.environ.pop("PAGED_ATTN_HEAD_PAIRS", None)
            else:
                os.environ["PAGED_ATTN_HEAD_PAIRS"] = env0
            forced = {k: rec[k + "_ms"] for k in ("one_S1", "one_S2", "pairs_S1", "pairs_S2")}
            best = min(forced, key=forced.get)
            rec.update({"best_forced": best, "plan_over_best": rec["plan_ms"] / forced[best]})
            emit(rec)
            del inp
            torch.cuda.empty_cache()
    elif name == "multitoken":
        # decode with q_len new tokens per sequence (speculative scoring): one
        # decode unit per sequence while q_len * G <= 16; HBM rate vs q_len = 1
        for hq, hkv, B, ctx, qls in ((32, 32, 64, 2048, (1, 2, 4, 8, 16)),
                                     (64, 8, 8, 16384, (1, 2))):
            for ql in qls:
                c = wl.multi_token_decode(B, ctx, ql, heads_q=hq, heads_kv=hkv,
                                          dtype="f16" if hq == hkv else "bf16")
                inp = wl.make_inputs(c, "cuda")
                S, med, mn = run(c, inp)
                by = algorithmic_bytes(c)
                emit({"sweep": "multitoken", "heads": f"{hq}/{hkv}", "batch": B, "ctx": ctx,
                      "q_len": ql, "splits": S, "ms": med, "ms_min": mn, "GBps": by / med / 1e6,
                      "frac": by / med / 1e6 / HBM_PEAK_GBS})
                del inp
                torch.cuda.empty_cache()
    elif name == "rotary":
        # the fused rotary embedding (q in the attention kernel, new keys in
        # the append kernel) against the same call without it
        points = (("mha_decode_b256_ctx4096_append", wl.mha_decode(256, 4096, append=True), 128),
                  ("gqa_long_split_paged", wl.gqa_long_split(True), 128),
                  ("causal_prefill_append_nq2048", wl.causal_prefill_append(2048, "zero"), 128),
                  ("unified_varlen_nq500_h32x128", wl.unified_varlen(500), 128),
                  ("unified_varlen_nq100_h12x64", wl.unified_varlen(100, heads=12, head_dim=64),
                   64))
        for label, c, rd in points:
            inp = wl.make_inputs(c, "cuda")
            cos, sin = wl.rotary_tables(max(c.keys_visible()) + 1, rd, c.dtype)
            res = {}
            for mode, rot in (("off", None), ("half_split", (cos, sin, False)),
                              ("interleaved", (cos, sin, True))):
                S, med, mn = run(c, inp, rot=rot)
                res[mode] = (med, mn)
            emit({"sweep": "rotary", "workload": label, "rotary_dim": rd, "splits": S,
                  "off_ms": res["off"][0], "half_split_ms": res["half_split"][0],
                  "interleaved_ms": res["interleaved"][0],
                  "overhead_half_split": res["half_split"][0] / res["off"][0] - 1.0,
                  "overhead_interleaved": res["interleaved"][0] / res["off"][0] - 1.0})
            del inp
            torch.cuda.empty_cache()
    elif name == "graph":
        # the same call eager and replayed from a HIP graph (launch overhead of
        # small, latency-bound calls); the buffers stay fixed, so one capture
        # replays the identical work
        points = (("mha_decode_b1_ctx512", wl.mha_decode(1, 512)),
                  ("mha_decode_b8_ctx1024", wl.mha_decode(8, 1024)),
                  ("unified_varlen_nq100_h12x64", wl.unified_varlen(100, heads=12, head_dim=64)))
        for label, c in points:
            inp = wl.make_inputs(c, "cuda")
            S, call = make_call(c, inp)
            call()
            torch.cuda.synchronize()
            e_med, e_min = median_call_ms(call, reps, torch, flush)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                call()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                call()
            torch.cuda.synchronize()
            g_med, g_min = median_call_ms(g.replay, reps, torch, flush)
            # back to back: 200 calls queued from Python, no flush - the
            # per-call rate when the host's launch cost is what limits
            loop = lambda fn: time_calls(fn, 200, 10, torch)
            emit({"sweep": "graph", "workload": label, "splits": S, "eager_ms": e_med,
                  "eager_ms_min": e_min, "graph_ms": g_med, "graph_ms_min": g_min,
                  "eager_loop_ms": loop(call), "graph_loop_ms": loop(g.replay)})
            del g, inp
            torch.cuda.empty_cache()
    fh.close()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--ctx", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the copy / GEMM ceiling measurements")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--sweep", choices=["copy", "decode", "gqa", "prefill", "unified", "graph", "rotary",
                                        "multitoken", "plan"],
                    help="run a measurement sweep instead of the headline line")
    ap.add_argument("--sweep-out", default="sweep.jsonl")
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()
    if args.sweep:
        sweep(args.sweep, args.reps, args.sweep_out)
        return
    if args.gpus != 1:
        print(f"bench.py: one GPU only; --gpus {args.gpus} is not supported (across GPUs the "
              "path would shard by sequence, kv head or key range, with no collective on it).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_lds_amd as pa
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.cuda.get_device_properties(0)
    log = lambda m: print(m, file=sys.stderr, flush=True)

    # ---- headline: MHA decode step (append + attend) ----
    case = wl.mha_decode(args.batch, args.ctx, page_size=16, append=True)
    case.causal = False
    log(f"bench: generating {case.name} on {dev.name}")
    inp = wl.make_inputs(case, "cuda")
    out = torch.empty_like(inp.q)
    lse = torch.empty(inp.q.shape[0], inp.q.shape[1], dtype=torch.float32, device="cuda")
    args_c = pa.make_args(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                          inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q,
                          max_seqlen_k=inp.max_seqlen_k, k_new=inp.k_new, v_new=inp.v_new,
                          out=out, softmax_lse=lse)
    splits = pa.paged_attn_splits_for(args_c)
    ws_bytes = pa.paged_attn_workspace_size(args_c)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        pa.paged_attn_fwd(inp.q, inp.k_cache, inp.v_cache, inp.block_table, inp.cache_seqlens,
                          inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q,
                          max_seqlen_k=inp.max_seqlen_k, k_new=inp.k_new, v_new=inp.v_new,
                          out=out, softmax_lse=lse, workspace=ws)

    log(f"bench: splits={splits}, timing {args.steps} steps after {args.warmup} warmup")
    torch.cuda.synchronize()
    ms = time_calls(step, args.steps, args.warmup, torch)
    step_bytes = algorithmic_bytes(case)
    value = step_bytes / (ms * 1e-3) / 1e9

    # ---- roofline of the attention kernel alone: same visible keys, no append ----
    seq_after = inp.cache_seqlens + 1          # the appended token is now in the cache
    attn_case = wl.Case(**{**case.__dict__, "append": False,
                           "cache_seqlens": [L + 1 for L in case.cache_seqlens]})

    def attn_only():
        pa.paged_attn_fwd(inp.q, inp.k_cache, inp.v_cache, inp.block_table, seq_after,
                          inp.cu_seqlens_q, max_seqlen_q=inp.max_seqlen_q,
                          max_seqlen_k=inp.max_seqlen_k, out=out, softmax_lse=lse, workspace=ws)

    attn_ms = time_calls(attn_only, args.steps, args.warmup, torch)
    attn_bytes = algorithmic_bytes(attn_case)
    achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(args.batch, args.ctx),
                "kernel": "attn_decode_kernel<f16,128>", "launch_ms": round(attn_ms, 4),
                "bytes_per_launch": attn_bytes, "splits": splits}

    # ---- CPU baseline: the oracle on a bounded sample of whole sequences ----
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        torch.cuda.synchronize()

        def sample(nseq):
            pages = [torch.from_numpy(np.asarray(inp.pages_of[b], dtype=np.int64)) for b in range(nseq)]
            flat = torch.cat(pages).cuda()
            kc = inp.k_cache.index_select(0, flat)
            vc = inp.v_cache.index_select(0, flat)
            width = max(len(p) for p in pages)
            table = np.full((nseq, width), -1, np.int32)
            off = 0
            for b, p in enumerate(pages):
                table[b, :len(p)] = np.arange(off, off + len(p))
                off += len(p)
            q = inp.q[:nseq]
            cu = np.arange(nseq + 1, dtype=np.int32)
            seq = np.asarray([L + 1 for L in case.cache_seqlens[:nseq]], np.int32)
            qh, kh, vh = wl.host(q), wl.host(kc), wl.host(vc)
            t0 = time.perf_counter()
            o, l = oracle.attention(qh, kh, vh, table, seq, cu, dtype="f16", appended=False,
                                    causal=False, threads=threads)
            return time.perf_counter() - t0, o, l

        t1, _, _ = sample(1)
        nseq = int(max(1, min(case.batch, args.cpu_seconds / max(t1, 1e-3))))
        log(f"bench: oracle on {nseq} sequences ({t1:.2f}s for one)")
        tc, o_ref, l_ref = sample(nseq)
        sub = wl.Case(**{**attn_case.__dict__, "q_lens": [1] * nseq,
                         "cache_seqlens": attn_case.cache_seqlens[:nseq]})
        cpu_gbs = algorithmic_bytes(sub) / tc / 1e9
        cpu_model = ""
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        cpu = {"value": round(cpu_gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "cpu_model": cpu_model,
               "sample": f"{nseq} of {case.batch} sequences (all 32 heads, {args.ctx + 1} keys "
                         f"each) of the same decode step, fp64 gather-then-softmax, "
                         f"{tc:.2f} s"}
        # sampled full-size parity: the attention-only output of those sequences
        attn_only()
        torch.cuda.synchronize()
        got = out[:nseq].float().cpu().numpy()
        err = float(np.abs(got - o_ref).max())
        lerr = float((np.abs(lse[:nseq].cpu().numpy() - l_ref) / np.abs(l_ref)).max())
        parity = {"rows": nseq * case.num_heads_q, "out_max_abs_err": err,
                  "lse_max_rel_err": lerr, "ok": bool(err <= 2e-3 and lerr <= 1e-4)}

    # ---- secondary: causal prefill with append ----
    prefill = None
    if not args.no_prefill:
        del inp
        torch.cuda.empty_cache()
        pc = wl.causal_prefill_append(2048, "zero")
        pin = wl.make_inputs(pc, "cuda")
        pout = torch.empty_like(pin.q)
        plse = torch.empty(pin.q.shape[0], pin.q.shape[1], dtype=torch.float32, device="cuda")

        def pstep():
            pa.paged_attn_fwd(pin.q, pin.k_cache, pin.v_cache, pin.block_table, pin.cache_seqlens,
                              pin.cu_seqlens_q, max_seqlen_q=pin.max_seqlen_q, k_new=pin.k_new,
                              v_new=pin.v_new, causal=True, out=pout, softmax_lse=plse)

        pms = time_calls(pstep, max(3, args.steps // 2), 2, torch)
        # the attention alone over the same keys (the appended rows are in the
        # pages by now): the prefill kernel without the append's copy
        seq_after = (pin.cache_seqlens + pc.q_lens[0]).contiguous()

        def pattn():
            pa.paged_attn_fwd(pin.q, pin.k_cache, pin.v_cache, pin.block_table, seq_after,
                              pin.cu_seqlens_q, max_seqlen_q=pin.max_seqlen_q, causal=True,
                              out=pout, softmax_lse=plse)

        ams = time_calls(pattn, max(3, args.steps // 2), 2, torch)
        fl = causal_flops(pc)
        tfs = fl / (pms * 1e-3) / 1e12
        atfs = fl / (ams * 1e-3) / 1e12
        prefill = {"workload": pc.name, "ms": round(pms, 4), "tflops": round(tfs, 2),
                   "peak": MFMA_F16_PEAK_TFS, "frac": round(tfs / MFMA_F16_PEAK_TFS, 4),
                   "attention_only_ms": round(ams, 4),
                   "attention_only_frac": round(atfs / MFMA_F16_PEAK_TFS, 4),
                   "flops_per_call": fl}

    # ---- measured references on this GPU: a large fp16 GEMM through the
    # vendor BLAS (what the MFMA units reach in practice, beside their peak)
    # and torch's device copy (read + write; torch's stream kernels stay well
    # below what a nontemporal read stream reaches, so it is no HBM ceiling) ----
    ceilings = None
    if not args.no_ceilings:
        torch.cuda.empty_cache()
        n = 1 << 30                                   # 2 GiB of fp16 read + 2 GiB written
        src = torch.empty(n, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        copy_ms = time_calls(lambda: dst.copy_(src), 10, 3, torch)
        del src, dst
        m = 8192
        a_ = torch.rand(m, m, dtype=torch.float16, device="cuda")
        b_ = torch.rand(m, m, dtype=torch.float16, device="cuda")
        gemm_ms = time_calls(lambda: torch.matmul(a_, b_), 10, 3, torch)
        del a_, b_
        copy_gbs = 4.0 * n / (copy_ms * 1e-3) / 1e9
        gemm_tfs = 2.0 * m ** 3 / (gemm_ms * 1e-3) / 1e12
        ceilings = {"gemm_f16_TFLOPs": round(gemm_tfs, 1),
                    "prefill_frac_of_gemm": (round(prefill["tflops"] / gemm_tfs, 4)
                                             if prefill else None),
                    "torch_copy_GBps": round(copy_gbs, 1)}

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": case.name + "_append1", "batch": case.batch,
                   "context": args.ctx, "heads_q": 32, "heads_kv": 32, "head_dim": 128,
                   "page_size": 16, "bytes_per_step": step_bytes, "splits": splits},
        "roofline": roofline, "cpu_baseline": cpu, "parity_sample": parity, "prefill": prefill,
        "ceilings": ceilings, "device": dev.name,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
