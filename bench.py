#!/usr/bin/env python3
"""Benchmark of the decode indexer path on one MI355X.

One step = one pass of the decode hot path over one batch:
  indexer_score_decode  (fused NVFP4 dequant + per-page scores, 4 requests x 8
                         query slots x 4 heads, 500,000-token contexts: 3,906
                         pages of 9,216 bytes per request)
  topk16_select         (the 128 score rows: 15 best pages below the own page,
                         then the own page)
Inputs are resident in HBM before timing starts.  The index-K cache rotates
over several independent pools (different layers in a real model) so that
their total exceeds the 256 MB last-level cache and every step streams from
HBM.

Prints one JSON line.  `value` is index-K bytes scored per second over the
whole step (GB/s); `roofline` reports the score kernel's own average launch
duration against the HBM peak; `cpu_baseline` is the CPU oracle timed on a
bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--pools P]
  python bench.py --workload decode-tiny|decode-mtp|decode-ragged   # the other decode batches
  python bench.py --profile-pass     # short fixed sequence for rocprofv3 counter runs
  python bench.py --workload prefill # lightning-indexer prefill step (scores + top-16)
  python bench.py --workload dequant # NVFP4 gather-dequantize of the decode pages
  python bench.py --workload nvfp4-prefill  # NVFP4 pages gathered, scored (4 heads), top-16
  python bench.py --workload mxfp8   # MXFP8 quantization of the attention output
  python bench.py --workload ragged-prefill  # causal ragged prefill (4 sequences, 64 heads)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "index-K GB/s scored (frac of HBM peak) + top-16 rows/s, 500K-token decode"
HBM_PEAK_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "score_decode_long_counters.txt")
SCORE_SOURCES = ["csrc/score_decode.hip", "csrc/wave_keys.hpp", "csrc/device_common.hpp",
                 "csrc/nvfp4_lut.hpp"]
MX_COUNTERS_FILE = os.path.join(ROOT, "profiles", "mxfp8_quant_counters.txt")
MX_SOURCES = ["csrc/mxfp8.hip", "csrc/device_common.hpp", "csrc/nvfp4_lut.hpp"]
DQ_COUNTERS_FILE = os.path.join(ROOT, "profiles", "nvfp4_dequant_counters.txt")
DQ_SOURCES = ["csrc/dequant.hip", "csrc/device_common.hpp", "csrc/nvfp4_lut.hpp"]
PREFILL_SOURCES = ["csrc/score_prefill.hip", "csrc/causal_share.hpp", "csrc/wave_keys.hpp",
                   "csrc/device_common.hpp", "csrc/nvfp4_lut.hpp"]
TOPK_SOURCES = ["csrc/topk16.hip", "csrc/wave_keys.hpp", "csrc/device_common.hpp", "csrc/nvfp4_lut.hpp"]


def _compile_flags(source):
    """hipcc flags of csrc/<source> from page_scoring_top_amd/build.py (loaded
    by path), without the machine-specific include paths."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_pagescore_build", os.path.join(ROOT, "page_scoring_top_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    flags = mod.common_flags() + mod.FILE_FLAGS.get(source, [])
    out, skip = [], False
    for f in flags:
        if skip:
            skip = False
        elif f == "-I":
            skip = True
        else:
            out.append(f)
    return out


def kernel_source_hash(sources=SCORE_SOURCES, flags_of="score_decode.hip") -> str:
    """Hash of a kernel's sources and compile flags (default: the decode scorer)."""
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "page_scoring_top_amd", f), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(_compile_flags(flags_of)).encode())
    return h.hexdigest()[:16]


def read_counters(path=COUNTERS_FILE, sources=SCORE_SOURCES, flags_of="score_decode.hip"):
    """HBM traffic per launch of a kernel from its committed rocprofv3 counter
    summary, or None when it is missing or the kernel changed since."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash(sources, flags_of):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--pools", type=int, default=None,
                    help="index-K pools rotated per step (default: per workload)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile-pass", action="store_true")
    ap.add_argument("--workload", choices=("decode", "decode-tiny", "decode-mtp", "decode-ragged",
                                           "prefill", "dequant", "nvfp4-prefill", "mxfp8",
                                           "ragged-prefill"),
                    default="decode")
    return ap.parse_args()


def timed(torch, stream, fn, n):
    """Average milliseconds per call of `fn` over `n` back-to-back calls, from
    two HIP events on the stream the kernels run on."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(n):
        fn(i)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / n


MFMA_F16_PEAK_TFLOPS = 2500.0


def bench_prefill(args):
    """Lightning-indexer prefill: 2,048 query tokens x 64 heads against 16,384
    keys, f32 scores, then the top-16 of every score row."""
    import torch

    import page_scoring_top_amd as ps
    import workloads

    dev = torch.device("cuda", 0)
    d = workloads.big_prefill()
    T, H = d.q.shape[0], d.q.shape[1]
    N = d.k.shape[0]
    q = torch.from_numpy(d.q).to(dev)
    qs = torch.from_numpy(d.q_scale).to(dev)
    k = torch.from_numpy(d.k).to(dev)
    ks = torch.from_numpy(d.k_scale).to(dev)
    scores = torch.zeros((T, N), dtype=torch.float32, device=dev)
    out = torch.zeros((T, 16), dtype=torch.int32, device=dev)
    score_call = ps.prepare(ps.indexer_score_prefill, q, qs, k, ks, scores)
    topk_call = ps.prepare(ps.topk16_select, scores, N, out)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        score_call()
        topk_call()
    torch.cuda.synchronize()
    K = args.steps

    def step(i):
        score_call()
        topk_call()

    clk = []
    step_st = windowed(torch, stream, step, K, clk)
    score_st = windowed(torch, stream, lambda i: score_call(), K, clk)
    topk_st = windowed(torch, stream, lambda i: topk_call(), K, clk)
    ms_per_step, score_ms, topk_ms = step_st["median"], score_st["median"], topk_st["median"]
    fused = fused_prefill_topk(torch, ps, stream, q, qs, k, ks, out, K, clk, ms_per_step)
    flops = 2.0 * T * N * H * 128          # the contraction (the epilogue is not counted)
    achieved = flops / (score_ms * 1e-3) / 1e12
    result = {
        "metric": "lightning-indexer prefill TFLOP/s (contraction) + top-16 rows/s",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3 values as f16, f32 accumulate", "data": "synthetic",
        "config": {"workload": "lightning-indexer prefill: 2,048 tokens x 64 heads x depth 128 "
                               "against 16,384 keys, then top-16 of 2,048 rows",
                   "tokens": T, "heads": H, "keys": N, "depth": 128, "parallelism": "single GPU"},
        "top16_rows_per_s": round(T / (topk_ms * 1e-3), 1),
        "timing": {"windows": WINDOWS, "step_us": us_stats(step_st)},
        "fused_top16": dict(fused, value=round(flops / (fused["step_us"]["median"] * 1e-6) / 1e12, 2),
                            unit="TFLOP/s"),
        "kernels_us": {"indexer_score_prefill": us_stats(score_st),
                       "topk16_select": us_stats(topk_st),
                       "timing": f"each kernel alone, median of {WINDOWS} windows of {K} launches",
                       "indexer_score_prefill_sustained": sustained_calls(torch, dev, [score_call])},
        "roofline": {"bound": "mfma", "kernel": "indexer_score_prefill",
                     "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops_per_launch": flops},
        "machine": machine_info(torch, clk),
    }
    if not args.no_cpu:
        import oracle
        t0 = time.perf_counter()
        n = 0
        while n < T and time.perf_counter() - t0 < args.cpu_seconds:
            oracle.score_prefill_rows(d.q, d.q_scale, d.k, d.k_scale, [n])
            n += 1
        t_rows = time.perf_counter() - t0
        cpu_step = t_rows * T / n
        result["cpu_baseline"] = {
            "value": round(flops / cpu_step / 1e12, 9), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"oracle prefill scores of {n} full rows ({t_rows:.2f} s), scaled to {T} rows; "
                      f"top-16 not included; step estimate {cpu_step:.1f} s"}
    print(json.dumps(result), flush=True)


def fused_prefill_topk(torch, ps, stream, q, qs, k, ks, chain_out, K, clk, chain_ms, before=None):
    """The same step with indexer_prefill_topk16 in place of the score matrix
    and topk16_select (after `before`, e.g. the gather, when given): its
    windows, the speed-up over the two-call step, and whether its output
    equals the two-call step's (run just before)."""
    T, N = q.shape[0], k.shape[0]
    ws = ps.prefill_topk16_workspace(T, N, q.device)
    out = torch.empty_like(chain_out)
    call = ps.prepare(ps.indexer_prefill_topk16, q, qs, k, ks, out, ws)

    def step(i):
        if before is not None:
            before()
        call()
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    same = bool(torch.equal(out, chain_out))
    st = windowed(torch, stream, step, K, clk)
    return {"call": "indexer_prefill_topk16", "step_us": us_stats(st),
            "speedup_vs_two_call_step": round(chain_ms / st["median"], 3),
            "matches_two_call_step": same, "workspace_bytes": int(ws.numel())}


def bench_ragged_prefill(args):
    """Ragged causal prefill: four sequences, each a 512-token chunk at the
    end of a 4,096 / 8,192 / 12,288 / 16,384-token context, 64 heads; scores
    masked causally with the -inf tail fill over a 16,384-column row, then
    the top-16 of every row over its visible keys."""
    import numpy as np
    import torch

    import page_scoring_top_amd as ps
    import workloads

    dev = torch.device("cuda", 0)
    d = workloads.ragged_prefill()
    T, H = d.p.q.shape[0], d.p.q.shape[1]
    W = d.width
    q = torch.from_numpy(d.p.q).to(dev)
    qs = torch.from_numpy(d.p.q_scale).to(dev)
    k = torch.from_numpy(d.p.k).to(dev)
    ks = torch.from_numpy(d.p.k_scale).to(dev)
    q_start = torch.from_numpy(d.q_start).to(dev)
    k_start = torch.from_numpy(d.k_start).to(dev)
    k_len = torch.from_numpy(d.k_len).to(dev)
    max_q = int(np.diff(d.q_start).max())
    scores = torch.empty((T, W), dtype=torch.float32, device=dev)
    row_len = torch.empty((T,), dtype=torch.int32, device=dev)
    out = torch.empty((T, 16), dtype=torch.int32, device=dev)
    score_call = ps.prepare(ps.indexer_score_prefill_ragged, q, qs, k, ks, q_start, k_start, k_len,
                            max_q, W, scores, row_len)
    topk_call = ps.prepare(ps.topk16_select, scores, W, out, valid_len=row_len)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        score_call()
        topk_call()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    clk = []
    step_st = windowed(torch, stream, step, K, clk)
    score_st = windowed(torch, stream, lambda i: score_call(), K, clk)
    topk_st = windowed(torch, stream, lambda i: topk_call(), K, clk)
    ms_per_step, score_ms, topk_ms = step_st["median"], score_st["median"], topk_st["median"]
    # Visible (query, key) pairs: sequence s's query i sees k_len - q_len + i + 1 keys.
    pairs = 0
    for s in range(len(d.k_len)):
        ql = int(d.q_start[s + 1] - d.q_start[s])
        kl = int(d.k_len[s])
        pairs += sum(min(max(kl - ql + i + 1, 0), min(kl, W)) for i in range(ql))
    flops = 2.0 * pairs * H * 128
    achieved = flops / (score_ms * 1e-3) / 1e12
    result = {
        "metric": "ragged causal lightning-indexer prefill TFLOP/s (visible pairs) + top-16",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3 values as f16, f32 accumulate", "data": "synthetic",
        "config": {"workload": "ragged causal prefill: 4 sequences x 512 query tokens x 64 heads "
                               "at 4,096-16,384-token contexts, rows of 16,384 columns with the "
                               "-inf tail fill, then top-16 of 2,048 rows",
                   "tokens": T, "heads": H, "width": W, "visible_pairs": pairs,
                   "parallelism": "single GPU"},
        "timing": {"windows": WINDOWS, "step_us": us_stats(step_st)},
        "kernels_us": {"indexer_score_prefill_ragged": us_stats(score_st),
                       "topk16_select": us_stats(topk_st),
                       "timing": f"each kernel alone, median of {WINDOWS} windows of {K} launches",
                       "indexer_score_prefill_ragged_sustained": sustained_calls(torch, dev,
                                                                                 [score_call])},
        "roofline": {"bound": "mfma", "kernel": "indexer_score_prefill_ragged",
                     "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops_per_launch": flops},
        "machine": machine_info(torch, clk),
    }
    if not args.no_cpu:
        import oracle
        t0 = time.perf_counter()
        n = 0
        order = [int(d.q_start[s]) + 3 * n_ % 512 for n_ in range(1000) for s in range(4)]
        done_pairs = 0
        while n < len(order) and time.perf_counter() - t0 < args.cpu_seconds:
            t = order[n]
            s = int(np.searchsorted(d.q_start, t, side="right") - 1)
            i = t - int(d.q_start[s])
            c = oracle.causal_count(int(d.q_start[s + 1] - d.q_start[s]), int(d.k_len[s]), i, W)
            k0 = int(d.k_start[s])
            oracle.score_prefill_rows(d.p.q, d.p.q_scale, d.p.k[k0:k0 + c], d.p.k_scale[k0:k0 + c],
                                      [t])
            done_pairs += c
            n += 1
        t_rows = time.perf_counter() - t0
        cpu_step = t_rows * pairs / max(done_pairs, 1)
        result["cpu_baseline"] = {
            "value": round(flops / cpu_step / 1e12, 9), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"oracle scores of {n} full visible rows ({done_pairs} pairs, {t_rows:.2f} s) "
                      f"spread over the four sequences, scaled to {pairs} pairs; top-16 not "
                      f"included; step estimate {cpu_step:.1f} s"}
    print(json.dumps(result), flush=True)


def bench_nvfp4_prefill(args):
    """Q8KV8 prefill chain: 512 NVFP4 pages (a 65,536-token context) gathered
    into E4M3 keys, 2,048 query tokens x 4 heads scored against them with unit
    key scales, then the top-16 of every score row."""
    import torch

    import page_scoring_top_amd as ps
    import workloads

    dev = torch.device("cuda", 0)
    d = workloads.nvfp4_prefill()
    T, H = d.q.shape[0], d.q.shape[1]
    N = int(d.context[0])
    P = d.total_pages
    kv = torch.from_numpy(d.kv_cache).to(dev)
    bt = torch.from_numpy(d.block_table).to(dev)
    num_pages = torch.from_numpy(d.num_pages).to(dev)
    offs = torch.from_numpy(d.page_offsets).to(dev)
    q = torch.from_numpy(d.q).to(dev)
    qs = torch.from_numpy(d.q_scale).to(dev)
    keys = torch.empty((P, 128, 128), dtype=torch.uint8, device=dev)
    ones = torch.ones(N, dtype=torch.float32, device=dev)
    scores = torch.empty((T, N), dtype=torch.float32, device=dev)
    out = torch.empty((T, 16), dtype=torch.int32, device=dev)
    gather_call = ps.prepare(ps.nvfp4_index_k_dequant, kv, bt, num_pages, offs,
                             d.block_table.shape[1], keys)
    score_call = ps.prepare(ps.indexer_score_prefill, q, qs, keys.view(-1, 128)[:N], ones, scores)
    topk_call = ps.prepare(ps.topk16_select, scores, N, out)
    if args.profile_pass:
        # Fixed sequence for counter runs: a plain 1 GiB device copy (the
        # calibration of FETCH_SIZE / WRITE_SIZE), then one launch of each call.
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        gather_call()
        score_call()
        topk_call()
        ws = ps.prefill_topk16_workspace(T, N, dev)
        ps.indexer_prefill_topk16(q, qs, keys.view(-1, 128)[:N], ones, out, ws)
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": True, "workload": "nvfp4-prefill", "copy_bytes": 1 << 30}),
              flush=True)
        return
    stream = torch.cuda.current_stream(dev)

    def step(i):
        gather_call()
        score_call()
        topk_call()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    clk = []
    step_st = windowed(torch, stream, step, K, clk)
    gather_st = windowed(torch, stream, lambda i: gather_call(), K, clk)
    score_st = windowed(torch, stream, lambda i: score_call(), K, clk)
    topk_st = windowed(torch, stream, lambda i: topk_call(), K, clk)
    ms_per_step, score_ms = step_st["median"], score_st["median"]
    fused = fused_prefill_topk(torch, ps, stream, q, qs, keys.view(-1, 128)[:N], ones, out, K, clk,
                               ms_per_step, before=gather_call)
    # Score kernel: queries, scales and keys read once, every score written once.
    algo = T * H * (128 + 4) + N * (128 + 4) + T * N * 4
    achieved = algo / (score_ms * 1e-3) / 1e9
    pairs = T * N
    result = {
        "metric": "NVFP4 (Q8KV8) prefill: query-key scores per second, gather + scores + top-16",
        "value": round(pairs / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "G scores/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3 values as f16, f32 accumulate", "data": "synthetic",
        "config": {"workload": "NVFP4 prefill: 512 pages (65,536-token context) gathered to E4M3, "
                               "2,048 tokens x 4 heads x depth 128 scored, top-16 of 2,048 rows",
                   "tokens": T, "heads": H, "keys": N, "pages": P, "parallelism": "single GPU"},
        "timing": {"windows": WINDOWS, "step_us": us_stats(step_st)},
        "fused_top16": dict(fused, value=round(pairs / (fused["step_us"]["median"] * 1e-6) / 1e9, 3),
                            unit="G scores/s"),
        "kernels_us": {"nvfp4_index_k_dequant": us_stats(gather_st),
                       "indexer_score_prefill": us_stats(score_st),
                       "topk16_select": us_stats(topk_st),
                       "timing": f"each kernel alone, median of {WINDOWS} windows of {K} launches",
                       "indexer_score_prefill_sustained": sustained_calls(torch, dev, [score_call])},
        "roofline": {"bound": "hbm", "kernel": "indexer_score_prefill",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": algo},
        "machine": machine_info(torch, clk),
    }
    if not args.no_cpu:
        import numpy as np
        import oracle
        t0 = time.perf_counter()
        keys_ora = oracle.gather(d.kv_cache, d.block_table, d.num_pages, d.page_offsets,
                                 d.block_table.shape[1],
                                 np.empty((P, 128, 128), dtype=np.uint8)).reshape(-1, 128)[:N]
        t_gather = time.perf_counter() - t0
        ones_h = np.ones(N, dtype=np.float32)
        t1 = time.perf_counter()
        n = 0
        oracle_rows = []
        while n < T and time.perf_counter() - t1 < args.cpu_seconds:
            row = oracle.score_prefill_rows(d.q, d.q_scale, keys_ora, ones_h, [n])
            oracle.topk16(row)
            oracle_rows.append(row[0])
            n += 1
        t_rows = time.perf_counter() - t1
        cpu_step = t_gather + t_rows * T / n
        # The GPU's scores of the same rows against the oracle's: the count
        # outside the plain bound 1e-6 + 1e-5 |oracle| (these cancelling dots
        # do not all meet it), and outside the same bound on the size of the
        # summed terms, M = sum_h q_scale sum_d |q k|.
        got = scores[:n].cpu().numpy().astype(np.float64)
        want = np.stack(oracle_rows).astype(np.float64)
        qa = torch.from_numpy(d.q[:n]).view(torch.float8_e4m3fn).double().abs()
        ka = torch.from_numpy(keys_ora).view(torch.float8_e4m3fn).double().abs()
        mag = (torch.matmul(qa, ka.T.contiguous()) *
               torch.from_numpy(d.q_scale[:n]).double().abs()[:, :, None]).sum(dim=1).numpy()
        err = np.abs(got - want)
        result["parity_sample"] = {
            "rows": n, "scores": int(want.size),
            "outside_plain_bound": int((err > 1e-6 + 1e-5 * np.abs(want)).sum()),
            "outside_term_bound": int((err > 1e-6 + 1e-5 * np.maximum(np.abs(want), mag)).sum())}
        result["cpu_baseline"] = {
            "value": round(pairs / cpu_step / 1e9, 9), "unit": "G scores/s", "cores": 1,
            "kind": "oracle",
            "sample": f"oracle gather of all {P} pages ({t_gather:.2f} s), then scores and top-16 "
                      f"of {n} full rows ({t_rows:.2f} s) scaled to {T} rows; "
                      f"step estimate {cpu_step:.1f} s"}
    print(json.dumps(result), flush=True)


def bench_mxfp8(args):
    """MXFP8 quantization of the attention output (the step after the sparse
    attention).  Timed: 16,384 rows x 2,048 bf16, a prefill-sized batch at
    one tensor-parallel rank's 2,048 columns, rotating over six independent
    input/output sets (610 MB, more than the 256 MB last-level cache) so each
    launch streams from HBM.  Also reported: the 128 x 2,048 decode batch
    (16 requests x 8 rows), which is launch-bound, timed as the pages time
    it: 200 launches captured in one HIP graph, median of 15 replays."""
    import torch

    import page_scoring_top_amd as ps
    import workloads

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    rows, cols, P = 16384, 2048, 6
    xh = workloads.mx_activations(5, rows, cols)
    calls = []
    for i in range(P):
        x = torch.from_numpy(xh.view("int16")).to(dev).view(torch.bfloat16)
        if i:
            x = x.roll(i, dims=0).contiguous()
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        sc = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        calls.append(ps.prepare(ps.mxfp8_e4m3_quantize, x, q, sc))
    if args.profile_pass:
        # Fixed sequence for counter runs: a plain 1 GiB device copy (the
        # calibration of FETCH_SIZE / WRITE_SIZE), then one launch per set.
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        for c in calls:
            c()
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": True, "copy_bytes": 1 << 30, "launches": P}), flush=True)
        return
    for i in range(args.warmup):
        calls[i % P]()
    torch.cuda.synchronize()
    clk = []
    st = windowed(torch, stream, lambda i: calls[i % P](), args.steps, clk)
    ms = st["median"]

    # Decode batch in a graph.
    dr = 128
    xd = torch.from_numpy(workloads.mx_activations(6, dr, cols).view("int16")).to(dev).view(
        torch.bfloat16)
    qd = torch.empty((dr, cols), dtype=torch.uint8, device=dev)
    sd = torch.empty((dr, cols // 32), dtype=torch.uint8, device=dev)
    ps.mxfp8_e4m3_quantize(xd, qd, sd)
    torch.cuda.synchronize()
    q_eager, s_eager = qd.clone(), sd.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(200):
                ps.mxfp8_e4m3_quantize(xd, qd, sd)
    torch.cuda.synchronize()
    reps = []
    for _ in range(15):
        qd.zero_()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        if not (torch.equal(qd, q_eager) and torch.equal(sd, s_eager)):
            raise RuntimeError("graph replay of mxfp8_e4m3_quantize differs from the eager result")
        reps.append(a.elapsed_time(b) / 200 * 1e3)
    decode_us = sorted(reps)[len(reps) // 2]

    algo = rows * cols * 3 + rows * cols // 32
    achieved = algo / (ms * 1e-3) / 1e9
    result = {
        "metric": "MXFP8 quantization of bf16 activations, GB/s (bytes in + out)",
        "value": round(achieved, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, e4m3 + e8m0 out",
        "data": "synthetic",
        "config": {"workload": "MXFP8 (E4M3 + E8M0 per 32) quantization of 16,384 x 2,048 bf16 "
                               "attention outputs, six rotating buffer sets",
                   "rows": rows, "cols": cols, "buffer_sets": P, "parallelism": "single GPU"},
        "kernels_us": {"mxfp8_e4m3_quantize": us_stats(st),
                       "timing": f"median of {WINDOWS} windows of {args.steps} launches",
                       "mxfp8_e4m3_quantize_sustained": sustained_calls(torch, dev, calls),
                       "mxfp8_e4m3_quantize_128x2048_graph": round(decode_us, 3)},
        "roofline": {"bound": "hbm", "kernel": "mxfp8_e4m3_quantize",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_counters(MX_COUNTERS_FILE, MX_SOURCES, "mxfp8.hip"),
                     "algorithmic_bytes_per_launch": algo},
        "machine": machine_info(torch, clk),
    }
    if not args.no_cpu:
        import oracle
        t0 = time.perf_counter()
        n = 0
        while n < rows and time.perf_counter() - t0 < args.cpu_seconds:
            oracle.mxfp8_quantize(xh[n:n + 64])
            n += 64
        t = time.perf_counter() - t0
        cpu_step = t * rows / n
        result["cpu_baseline"] = {
            "value": round(algo / cpu_step / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle quantization of {n} rows ({t:.2f} s), scaled to {rows} rows"}
    print(json.dumps(result), flush=True)


def bench_dequant(args):
    """Gather-dequantize of every scored page of the 500K-token decode batch
    (15,624 pages) into contiguous E4M3 pages, rotating over index-K pools."""
    import torch

    import page_scoring_top_amd as ps
    import workloads

    dev = torch.device("cuda", 0)
    d = workloads.long_decode()
    R, W = d.num_reqs, d.width
    P = max(1, args.pools if args.pools is not None else 4)
    pools = [torch.from_numpy(d.kv_cache).to(dev)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    for _ in range(1, P):
        kv = torch.empty_like(pools[0])
        kv[:, :8192] = torch.randint(0, 256, (kv.shape[0], 8192), generator=gen, device=dev,
                                     dtype=torch.uint8)
        kv[:, 8192:] = torch.randint(1, 127, (kv.shape[0], 1024), generator=gen, device=dev,
                                     dtype=torch.uint8)
        pools.append(kv)
    bt = torch.from_numpy(d.block_table[:R]).to(dev)
    npages = [min(max((int(s) - 1) // 128, 0), W) for s in d.seq_lens[:R]]
    num_pages = torch.tensor(npages, dtype=torch.int32, device=dev)
    offs = torch.tensor([sum(npages[:i]) for i in range(R)], dtype=torch.int32, device=dev)
    total = sum(npages)
    out = torch.empty((total, 128, 128), dtype=torch.uint8, device=dev)
    calls = [ps.prepare(ps.nvfp4_index_k_dequant, kv, bt, num_pages, offs, W, out) for kv in pools]
    if args.profile_pass:
        # Counter runs: the 1 GiB calibration copy, then one launch per pool.
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        for c in calls:
            c()
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": True, "copy_bytes": 1 << 30, "launches": P}), flush=True)
        return
    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        calls[i % P]()
    torch.cuda.synchronize()
    K = args.steps
    clk = []
    st = windowed(torch, stream, lambda i: calls[i % P](), K, clk)
    ms = st["median"]
    algo = total * (9216 + 4 + 16384) + R * 8
    achieved = algo / (ms * 1e-3) / 1e9
    result = {
        "metric": "NVFP4 index-K gather-dequantize GB/s (bytes in + out)",
        "value": round(achieved, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8 (e4m3 bytes out)", "data": "synthetic",
        "config": {"workload": "gather-dequantize of the 500K-token decode batch: 4 requests x "
                               "3,906 NVFP4 pages into contiguous E4M3 pages",
                   "pages": total, "index_k_pools": P, "parallelism": "single GPU"},
        "kernels_us": {"nvfp4_index_k_dequant": us_stats(st),
                       "timing": f"median of {WINDOWS} windows of {K} launches",
                       "nvfp4_index_k_dequant_sustained": sustained_calls(torch, dev, calls)},
        "roofline": {"bound": "hbm", "kernel": "nvfp4_index_k_dequant",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_counters(DQ_COUNTERS_FILE, DQ_SOURCES, "dequant.hip"),
                     "algorithmic_bytes_per_launch": algo},
        "machine": machine_info(torch, clk),
    }
    if not args.no_cpu:
        import numpy as np
        import oracle
        t0 = time.perf_counter()
        n = 0
        ids = d.block_table[0]
        while n < total and time.perf_counter() - t0 < args.cpu_seconds:
            oracle.dequant_page(d.kv_cache[ids[n % W]])
            n += 1
        t = time.perf_counter() - t0
        cpu_step = t * total / n
        result["cpu_baseline"] = {
            "value": round(algo / cpu_step / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle dequantization of {n} pages ({t:.2f} s), scaled to {total} pages"}
        del np
    print(json.dumps(result), flush=True)


# Inputs of the oracle's worker processes, set before they are forked.
_CPU_DECODE = None


def _decode_page(d, W, p):
    """The step's scored page p as (request, column): requests in order, each
    with its scored columns 0 .. pages_scored - 1."""
    for b in range(d.num_reqs):
        n = min(max((int(d.seq_lens[b]) - 1) // 128, 0), W)
        if p < n:
            return b, p
        p -= n
    raise IndexError(p)


def _oracle_decode_worker(w, workers, seconds):
    """Worker w of `workers`: oracle decode scores (all 32 rows of the page's
    request) of the step's pages w, w + workers, ... until `seconds` pass;
    (pages, seconds)."""
    import oracle
    d, qlen, W, pages = _CPU_DECODE
    t0 = time.perf_counter()
    n = 0
    p = w
    while p < pages and time.perf_counter() - t0 < seconds:
        b, j = _decode_page(d, W, p)
        oracle.score_decode_column(d.kv_cache, d.block_table, d.seq_lens, d.q, d.q_scale, qlen, W,
                                   b, j)
        n += 1
        p += workers
    return n, time.perf_counter() - t0


def host_cores() -> int:
    """This process's CPU share, at most 16 (the share of one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_decode_parallel(d, qlen, W, pages, seconds):
    """The oracle's decode scoring rate (pages/s) over forked worker processes,
    one per host core of this process's share (at most 16).  Runs before the
    GPU is initialized, so the fork copies no GPU state."""
    import multiprocessing as mp

    import oracle
    global _CPU_DECODE
    oracle.lib()                       # built and loaded once, before the fork
    _CPU_DECODE = (d, qlen, W, pages)
    workers = min(host_cores(), pages)
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.starmap(_oracle_decode_worker, [(w, workers, seconds) for w in range(workers)])
    n = sum(r[0] for r in res)
    t = max(r[1] for r in res)
    return n, t, workers


def decode_pages_of(d):
    return sum(min(max((int(s) - 1) // 128, 0), d.width) for s in d.seq_lens[:d.num_reqs])


def oracle_decode_legs(d, seconds):
    """The oracle on a decode step, on one core and on one process per core:
    pages per second of full-page scoring (all 32 rows of a page's request)
    and the time of its top-16 over the step's rows (seeded N(0,1) rows of the
    step's width, with the rows' own pages as valid lengths and appended
    pages)."""
    import numpy as np

    import oracle
    W = d.width
    pages = decode_pages_of(d)
    t0 = time.perf_counter()
    n = 0
    stride = 7   # pages spread over the step's requests
    while n < pages and time.perf_counter() - t0 < seconds:
        b, j = _decode_page(d, W, (n * stride) % pages)
        oracle.score_decode_column(d.kv_cache, d.block_table, d.seq_lens, d.q, d.q_scale, d.qlen,
                                   W, b, j)
        n += 1
    t_cols = time.perf_counter() - t0
    rows = np.random.default_rng(7).standard_normal((d.num_reqs * 32, W)).astype(np.float32)
    own = np.array([min(max((int(d.seq_lens[b]) - 1) // 128, 0), W) for b in range(d.num_reqs)
                    for _ in range(32)], dtype=np.int32)
    t1 = time.perf_counter()
    oracle.topk16(rows, own, None, None, own)
    t_topk = time.perf_counter() - t1
    pn, pt, workers = oracle_decode_parallel(d, d.qlen, W, pages, seconds)
    return {"pages": pages, "single": (n, t_cols), "parallel": (pn, pt, workers), "topk_s": t_topk}


# ---------------------------------------------------------------------------
# Timing helpers shared by the decode legs.
# ---------------------------------------------------------------------------

WINDOWS = 7            # repeated timed windows; the median is reported
GRAPH_STEPS = 200      # steps captured per HIP graph
GRAPH_REPLAYS = 15     # replays of it; the median is reported


def stats(values):
    v = sorted(values)
    med = v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
    return {"median": med, "min": v[0], "max": v[-1],
            "spread": (v[-1] - v[0]) / med if med > 0 else None}


def windowed(torch, stream, fn, n, clk):
    """Statistics (ms per call) of WINDOWS windows of `n` back-to-back calls,
    reading the shader clock into `clk` while each window runs."""
    return stats([timed_sampling_clock(torch, stream, fn, n, clk) for _ in range(WINDOWS)])


def us_stats(st):
    """A stats() dict in microseconds (the spread stays a fraction)."""
    return {k: (round(v * 1e3, 3) if k != "spread" else round(v, 4)) for k, v in st.items()}


def _capture(torch, dev, make_step, steps):
    """One HIP graph holding `steps` steps; `make_step()` builds the step's
    calls on the current (capture) stream."""
    stream = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step = make_step()
        step(0)                          # built and run once on the side stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                step(i)
    torch.cuda.synchronize()
    return g


def graph_replay_ms(torch, dev, make_step, steps=GRAPH_STEPS, replays=GRAPH_REPLAYS):
    """Median ms per step of `steps` steps captured in one HIP graph and
    replayed `replays` times (the pages' own timing method)."""
    stream = torch.cuda.current_stream(dev)
    g = _capture(torch, dev, make_step, steps)
    g.replay()                           # warm
    torch.cuda.synchronize()
    per = []
    for _ in range(replays):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / steps)
    del g
    return stats(per)


def _sclk_mhz(torch):
    """The GPU's current shader clock from sysfs (pp_dpm_sclk, the level
    marked '*'), or None where it cannot be read."""
    try:
        p = torch.cuda.get_device_properties(0)
        path = f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:" \
               f"{p.pci_device_id:02x}.0/pp_dpm_sclk"
        for line in open(path):
            if "*" in line:
                return float(line.split(":")[1].strip().split("M")[0].rstrip("*").strip())
    except Exception:
        return None
    return None


def _hwmon(torch, name):
    """A value of the GPU's hwmon node (microwatts for power files), or None."""
    import glob
    try:
        p = torch.cuda.get_device_properties(0)
        base = f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:" \
               f"{p.pci_device_id:02x}.0/hwmon/hwmon*/{name}"
        for path in sorted(glob.glob(base)):
            return float(open(path).read().split()[0])
    except Exception:
        return None
    return None


def sustained_power(torch, dev, make_step, seconds=1.0, steps=GRAPH_STEPS):
    """Board power while the step runs back to back for about `seconds`
    (HIP-graph replays, no host gaps), read from hwmon every 2 ms on a host
    thread; the first quarter of the samples (ramp) is dropped.  Returns the
    median power, the board's power cap and the time per step meanwhile, or
    None where the power cannot be read."""
    import threading
    import time
    if _hwmon(torch, "power1_input") is None:
        return None
    stream = torch.cuda.current_stream(dev)
    g = _capture(torch, dev, make_step, steps)
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    per_replay = max(time.perf_counter() - t0, 1e-4)
    n = max(4, int(seconds / per_replay))
    samples, run = [], [True]

    def sample():
        while run[0]:
            samples.append(_hwmon(torch, "power1_input"))
            time.sleep(0.002)
    th = threading.Thread(target=sample)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    th.start()
    a.record(stream)
    for _ in range(n):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    run[0] = False
    th.join()
    del g
    got = [v for v in samples[len(samples) // 4:] if v is not None]
    cap = _hwmon(torch, "power1_cap")
    return {"power_w": round(stats(got)["median"] / 1e6, 1) if got else None,
            "power_cap_w": round(cap / 1e6, 1) if cap else None,
            "us_per_step": round(a.elapsed_time(b) * 1e3 / (n * steps), 3),
            "seconds": round(a.elapsed_time(b) / 1e3, 3), "samples": len(got)}


def sustained_calls(torch, dev, calls):
    """sustained_power() of prepared calls taken in turn, one per step."""
    def make():
        cs = [c.again() for c in calls]
        return lambda i: cs[i % len(cs)]()
    return sustained_power(torch, dev, make)


def machine_info(torch, sclk_samples):
    """Which machine ran: host name, device identity, the peak shader clock
    the runtime reports, and the shader clock read while timed work ran."""
    import ctypes
    import socket
    p = torch.cuda.get_device_properties(0)
    info = {"host": socket.gethostname(), "gpu": p.name, "arch": p.gcnArchName,
            "compute_units": p.multi_processor_count, "uuid": str(p.uuid),
            "pci": f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:   # hipDeviceAttributeClockRate
            info["peak_sclk_mhz"] = v.value / 1000.0
    except OSError:
        pass
    got = [s for s in sclk_samples if s is not None]
    info["sclk_mhz_during_timing"] = stats(got) if got else None
    return info


def timed_sampling_clock(torch, stream, fn, n, samples):
    """timed(), reading the shader clock while the launched work runs."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(n):
        fn(i)
    stop.record(stream)
    samples.append(_sclk_mhz(torch))
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / n


# ---------------------------------------------------------------------------
# Decode legs.
# ---------------------------------------------------------------------------

# Index-K pools per leg: enough that the pools rotated through a timed window
# exceed the 256 MB last-level cache (at least 512 MB in total), except the
# tiny batch, which is latency-bound and cache-resident by nature.
DECODE_LEGS = {
    "decode": ("long_decode", 4,
               "long-context decode: 4 requests x 8 query slots x 4 index heads, 500,000-token "
               "contexts (3,906 NVFP4 pages scored per request), then top-16 of 128 score rows"),
    "decode-tiny": ("tiny_decode", 1,
                    "tiny decode: 1 request, 1 query token x 4 index heads, 8,192-token context "
                    "(63 NVFP4 pages scored), then top-16 of its 4 score rows"),
    "decode-mtp": ("mtp_decode", 15,
                   "MTP decode: 16 requests x 8 query slots x 4 index heads, 30,000-token "
                   "contexts (234 NVFP4 pages scored per request), then top-16 of 512 rows"),
    "decode-ragged": ("ragged_decode", 2,
                      "ragged decode: 64 requests x 8 query slots x 4 index heads, contexts "
                      "uniform in 1,000-172,032 tokens, rows of 1,344 columns, 8 padding "
                      "requests, then top-16 of 2,048 rows"),
}


def bench_decode(args, leg, cpu_legs):
    import torch

    import page_scoring_top_amd as ps
    import workloads

    dev = torch.device("cuda", 0)
    maker, default_pools, workload = DECODE_LEGS[leg]
    d = getattr(workloads, maker)()
    R, W, qlen = d.num_reqs, d.width, d.qlen
    Rt = d.q.shape[0]
    P = max(1, args.pools if args.pools is not None else default_pools)

    # Index-K pools: pool 0 is the seeded host workload; the others are drawn
    # on the device with their own seeded generator (same distributions:
    # uniform code bytes, scale bytes uniform over 0x01..0x7E).
    pools = [torch.from_numpy(d.kv_cache).to(dev)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    for _ in range(1, P):
        kv = torch.empty_like(pools[0])
        kv[:, :8192] = torch.randint(0, 256, (kv.shape[0], 8192), generator=gen, device=dev,
                                     dtype=torch.uint8)
        kv[:, 8192:] = torch.randint(1, 127, (kv.shape[0], 1024), generator=gen, device=dev,
                                     dtype=torch.uint8)
        pools.append(kv)
    bt = torch.from_numpy(d.block_table).to(dev)
    seq = torch.from_numpy(d.seq_lens).to(dev)
    q = torch.from_numpy(d.q).to(dev)
    qs = torch.from_numpy(d.q_scale).to(dev)
    scores = torch.zeros((Rt, 32, W), dtype=torch.float32, device=dev)
    own = torch.zeros((Rt, 32), dtype=torch.int32, device=dev)
    out = torch.zeros((R * 32, 16), dtype=torch.int32, device=dev)

    def make_calls():
        sc = [ps.prepare(ps.indexer_score_decode, kv, bt, seq, q, qs, qlen, W, scores, own,
                         num_reqs=R) for kv in pools]
        tk = ps.prepare(ps.topk16_select, scores[:R].view(R * 32, W), W, out,
                        valid_len=own[:R].view(-1), append_page=own[:R].view(-1))
        return sc, tk

    score_calls, topk_call = make_calls()
    pages = decode_pages_of(d)
    kbytes = pages * 9216
    stored = 0
    for b in range(R):
        npg = min(max((int(d.seq_lens[b]) - 1) // 128, 0), W)
        for slot in range(8):
            i = slot - (8 - qlen)
            pos = int(d.seq_lens[b]) - qlen + i
            own_p = pos // 128 if i >= 0 and pos >= 0 else -1
            stored += 4 * min(max(own_p, 0), npg)
    # Algorithmic bytes of one score launch: index-K pages, their block-table
    # entries, score writes, and per request q, q_scale, seq_len and own pages.
    algo_bytes = pages * (9216 + 4) + stored * 4 + R * (4096 + 128 + 4 + 128)

    if args.profile_pass:
        # Fixed sequence for counter runs: a plain 1 GiB device copy (the
        # calibration of FETCH_SIZE / WRITE_SIZE), then one score launch per
        # pool and one top-16.
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        for c in score_calls:
            c()
        topk_call()
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": True, "workload": leg, "copy_bytes": 1 << 30,
                          "score_launches": P, "score_algo_bytes": algo_bytes}), flush=True)
        return

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        score_calls[i % P]()
        topk_call()
    torch.cuda.synchronize()

    def step(i):
        score_calls[i % P]()
        topk_call()

    K = args.steps
    clk = []
    # The timed region: windows of K whole steps back to back; the median
    # window is reported.
    step_ms = stats([timed_sampling_clock(torch, stream, step, K, clk) for _ in range(WINDOWS)])

    # The same step, and each kernel alone, as HIP-graph replays: no host
    # launch cost between kernels, so a small kernel's time is its own (a
    # back-to-back loop of small kernels measures the host's launch rate).
    def make_step():
        sc, tk = make_calls()

        def graph_step(i):
            sc[i % P]()
            tk()
        return graph_step

    def make_score():
        sc, _ = make_calls()
        return lambda i: sc[i % P]()

    def make_topk():
        _, tk = make_calls()
        return lambda i: tk()

    graph_ms = graph_replay_ms(torch, dev, make_step)
    score_ms = graph_replay_ms(torch, dev, make_score)
    topk_ms = graph_replay_ms(torch, dev, make_topk)
    # The score kernel for about a second, with the board's power read meanwhile.
    score_power = sustained_power(torch, dev, make_score)
    # The score kernel alone, back to back with HIP events (host-launched).
    score_loop_ms = stats([timed_sampling_clock(torch, stream, lambda i: score_calls[i % P](), K, clk)
                           for _ in range(WINDOWS)])

    ms_per_step = step_ms["median"]
    value = kbytes / (ms_per_step * 1e-3) / 1e9
    achieved = algo_bytes / (score_ms["median"] * 1e-3) / 1e9
    traffic = read_counters(counters_file(leg))

    us = us_stats

    result = {
        "metric": METRIC if leg == "decode" else
        f"index-K GB/s scored (frac of HBM peak) + top-16 rows/s, {leg[7:]} decode",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 values as f16, f32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "requests": R, "query_slots": 8, "qlen": qlen, "heads": 4, "depth": 128,
            "seq_len": int(d.seq_lens[0]) if leg != "decode-ragged" else "1,000-172,032",
            "pages_scored": pages, "index_k_bytes": kbytes, "width": W, "index_k_pools": P,
            "parallelism": "single GPU",
        },
        "top16_rows_per_s": round(R * 32 / (topk_ms["median"] * 1e-3), 1),
        "timing": {
            "windows": WINDOWS,
            "step_us": us(step_ms),
            "graph_replay_step_us": us(graph_ms),
            "graph_replay": f"{GRAPH_STEPS} steps per HIP graph, median of {GRAPH_REPLAYS} "
                            f"replays",
            "graph_value": round(kbytes / (graph_ms["median"] * 1e-3) / 1e9, 2),
        },
        "kernels_us": {"indexer_score_decode": us(score_ms), "topk16_select": us(topk_ms),
                       "timing": f"each kernel alone, {GRAPH_STEPS} launches per HIP graph, median of "
                                 f"{GRAPH_REPLAYS} replays",
                       "indexer_score_decode_host_loop": us(score_loop_ms),
                       "indexer_score_decode_sustained": score_power},
        "roofline": {
            "bound": "hbm",
            "kernel": "indexer_score_decode",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": algo_bytes,
        },
        "machine": machine_info(torch, clk),
    }

    if cpu_legs is not None:
        n, t_cols = cpu_legs["single"]
        pn, pt, workers = cpu_legs["parallel"]
        t_topk = cpu_legs["topk_s"]
        step1 = t_cols * pages / n + t_topk
        stepn = pt * pages / pn + t_topk
        result["cpu_baseline"] = {
            "value": round(kbytes / stepn / 1e9, 6),
            "unit": "GB/s",
            "cores": workers,
            "kind": "oracle",
            "sample": f"the oracle in {workers} worker processes (one per host core of this "
                      f"process): {pn} full pages (32 rows each) in {pt:.2f} s, scaled to "
                      f"{pages} pages, plus the single-core oracle top-16 of {R * 32} rows of "
                      f"width {W} ({t_topk:.3f} s); step estimate {stepn:.2f} s",
        }
        result["cpu_baseline_1core"] = {
            "value": round(kbytes / step1 / 1e9, 6),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"the oracle on one core: {n} full pages in {t_cols:.2f} s, scaled to "
                      f"{pages} pages, plus the same top-16; step estimate {step1:.2f} s",
        }
    print(json.dumps(result), flush=True)


def counters_file(leg):
    """The committed FETCH/WRITE counter summary of a decode leg."""
    name = {"decode": "long", "decode-tiny": "tiny", "decode-mtp": "mtp",
            "decode-ragged": "ragged"}[leg]
    return os.path.join(ROOT, "profiles", f"score_decode_{name}_counters.txt")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the indexer path "
                          "has no multi-GPU mode", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    # The parallel oracle leg of a decode step forks worker processes, so it
    # runs before anything touches the GPU.
    cpu_legs = None
    if args.workload in DECODE_LEGS and not args.no_cpu and not args.profile_pass:
        import workloads
        d = getattr(workloads, DECODE_LEGS[args.workload][0])()
        cpu_legs = oracle_decode_legs(d, args.cpu_seconds)
        del d

    import torch
    torch.cuda.set_device(0)
    if args.workload == "prefill":
        return bench_prefill(args)
    if args.workload == "dequant":
        return bench_dequant(args)
    if args.workload == "nvfp4-prefill":
        return bench_nvfp4_prefill(args)
    if args.workload == "mxfp8":
        return bench_mxfp8(args)
    if args.workload == "ragged-prefill":
        return bench_ragged_prefill(args)
    return bench_decode(args, args.workload, cpu_legs)


if __name__ == "__main__":
    main()
