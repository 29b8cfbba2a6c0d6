"""Benchmark: Spava / APB-V approximate-attention prefill on one MI355X.

One step = the whole hot path on one batch of synthetic input already resident in
HBM: passing-block selection (fp64 scores + top-l) followed by the approximate
attention (gather + schedule + bf16 MFMA attention). Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload h8_128k]

`value` is prefill tokens/s (N / step time). `tflops` counts the algorithmic
attention FLOPs (4 * d * Hq * key-visits over the approximate visible sets, causal
triangle exact) divided by the attention call's time. `roofline` reports that
attention call against the bf16 dense MFMA peak; `cpu_baseline` times the fp64
oracle on a bounded sample on the host cores and extrapolates by work.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "approx-attn prefill tokens/s + TFLOP/s (% bf16 MFMA peak), 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA (published)
PEAK_CLOCK_GHZ = 2.4                # the clock the published peak assumes
PMC_SUMMARY = os.path.join(ROOT, "profiles", "attn_bf16_{workload}_pmc.json")
ATTN_SOURCES = [os.path.join(ROOT, "long_context_approximate_amd", "csrc", f)
                for f in ("attn_bf16.hip", "attn_common.h")]


def key_visits_per_head(cfg) -> int:
    """Sum over blocks h and their queries i of |V(i)| = L_h + (i - s_h + 1)."""
    nb, H, A, l = cfg.block_len, cfg.num_hosts, cfg.anchor_len, cfg.passing_len
    l0 = min(l, nb - A) if H > 1 else 0
    l1 = min(l, nb)
    total = 0
    for h in range(H):
        L = 0 if h == 0 else A + l0 + (h - 1) * l1
        total += nb * (nb + 1) // 2 + nb * L
    return total


def attn_flops(cfg) -> float:
    return 4.0 * cfg.head_dim * cfg.num_q_heads * key_visits_per_head(cfg)


def attn_sources_sha256() -> str:
    """Hash of the attention kernel's source code (the counters are tied to it): the
    files with `//` comments, trailing blanks and empty lines removed, so that editing
    a comment does not mark the profiles stale."""
    h = hashlib.sha256()
    for path in ATTN_SOURCES:
        for line in open(path, encoding="utf-8").read().splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def _profile_field(workload, *keys):
    """A number from the committed rocprofv3 counter summary of this workload, or None
    when the summary is missing, lacks the field, or the attention source changed since
    it was taken."""
    try:
        rec = json.load(open(PMC_SUMMARY.format(workload=workload)))
        if rec.get("attn_sources_sha256") != attn_sources_sha256():
            return None
        for k in keys:
            rec = rec[k]
        return float(rec)
    except (OSError, ValueError, KeyError, TypeError):
        return None


def clock_from_profile(workload):
    """Average shader clock (GHz) during the attention kernel (GRBM_GUI_ACTIVE run)."""
    return _profile_field(workload, "attn_clock_ghz")


def traffic_from_profile(workload):
    """HBM bytes per attention launch (FETCH_SIZE + WRITE_SIZE runs, calibrated)."""
    return _profile_field(workload, "hbm_bytes_per_launch")


def score_flops(cfg) -> float:
    """fp64 FLOP of the window-score dot products: 2 d per (observer row, visible key);
    row i of the last w of a block sees the block's keys up to i."""
    H, hkv, G = cfg.num_hosts, cfg.num_kv_heads, cfg.num_q_heads // cfg.num_kv_heads
    nb, w = cfg.seq_len // H, cfg.window
    visits = w * nb - w * (w - 1) // 2
    return 2.0 * cfg.head_dim * max(H - 1, 0) * hkv * G * visits


def _oracle_sample(cfg, x, budget_rows, pairs_sampled):
    """Time the fp64 oracle on a sample of the workload and extrapolate to the whole.

    Sample: the window scores + top-l of `pairs_sampled` (block, KV head) pairs, and
    `budget_rows` query rows of one head in the first, a middle and the last block.
    The whole-workload time is extrapolated pair-by-pair for selection and by the
    oracle's own per-row key count (L_h + n_b keys per row) for attention.
    Returns (estimated seconds for the whole workload, measured seconds, description).
    """
    import numpy as np

    import oracle
    sh = oracle.shape_of(cfg)
    nb, H = cfg.block_len, cfg.num_hosts
    pairs = max(H - 1, 0) * cfg.num_kv_heads
    n_pairs = min(pairs_sampled, pairs)
    t0 = time.perf_counter()
    for pi in range(n_pairs):
        j, g = divmod(pi, cfg.num_kv_heads)
        sc = oracle.window_scores(sh, x["q"], x["k"], j, g)
        order = np.lexsort((np.arange(nb), -sc))[: cfg.passing_len]
        del order
    t_pair = (time.perf_counter() - t0) / max(n_pairs, 1)
    idx = np.full((max(H - 1, 0), cfg.num_kv_heads, cfg.passing_len), -1, np.int32)
    for j in range(H - 1):       # a valid selection pattern of the right size
        cand = oracle.passing_candidates(sh, j)
        lj = oracle.passing_length(sh, j)
        idx[j, :, :lj] = cand[:lj]
    sample_cost = 0.0
    t_rows = 0.0
    blocks = sorted({0, H // 2, H - 1})
    for h in blocks:
        s = h * nb
        rows = np.arange(s, s + min(budget_rows, nb))
        L = len(oracle.visible_prefix(sh, idx, h, 0))
        t1 = time.perf_counter()
        oracle.attention_rows(sh, x["q"], x["k"], x["v"], idx, 0, rows)
        t_rows += time.perf_counter() - t1
        sample_cost += len(rows) * (L + nb)
    total_cost = 0.0
    for h in range(H):
        L = len(oracle.visible_prefix(sh, idx, h, 0))
        total_cost += nb * (L + nb) * cfg.num_q_heads
    t_total = t_pair * pairs + t_rows * (total_cost / sample_cost)
    measured = t_pair * n_pairs + t_rows
    desc = (f"window scores + top-l of {n_pairs} of {pairs} (block, kv-head) pairs, and "
            f"{min(budget_rows, nb)} query rows x 1 head in blocks {blocks}; extrapolated by "
            f"pair count and by the oracle's per-row key count (measured {measured:.1f} s)")
    return t_total, measured, desc


def _blas_info():
    """BLAS libraries numpy runs on and their thread counts (threadpoolctl)."""
    try:
        import numpy  # noqa: F401  (loads the BLAS threadpoolctl inspects)
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        return {"blas": "unknown", "blas_threads": 1}
    names = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in libs})
    threads = max([int(i.get("num_threads", 1)) for i in libs] or [1])
    return {"blas": ", ".join(names) or "none", "blas_threads": threads}


def _single_core_oracle():
    """The oracle on one host thread for the two smallest workloads: the 512-token one
    in full (measured), the 16K one from a bounded sample (extrapolated)."""
    import oracle
    from long_context_approximate_amd.inputs import CONFIGS, make_inputs
    out = {}
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        return None
    with threadpool_limits(limits=1):
        tiny = CONFIGS["tiny_f32_512"]
        xt = make_inputs(tiny)
        t0 = time.perf_counter()
        oracle.run(oracle.shape_of(tiny), xt["q"], xt["k"], xt["v"])
        dt = time.perf_counter() - t0
        out[tiny.name] = {"seconds": dt, "tokens_per_s": tiny.seq_len / dt, "kind": "measured",
                          "sample": "the whole workload (selection + attention)"}
        c2 = CONFIGS["h4_16k"]
        x2 = make_inputs(c2)
        est, measured, desc = _oracle_sample(c2, x2, budget_rows=4096, pairs_sampled=2)
        out[c2.name] = {"seconds": est, "tokens_per_s": c2.seq_len / est,
                        "kind": "extrapolated", "sample": desc}
    return out


def cpu_baseline(cfg, x, budget_rows=16384, pairs_sampled=8):
    """The fp64 oracle on the host cores: a bounded sample of the benchmarked workload,
    extrapolated (see _oracle_sample), with the BLAS it ran on, plus one-thread times of
    the two smallest workloads."""
    est, measured, desc = _oracle_sample(cfg, x, budget_rows, pairs_sampled)
    blas = _blas_info()
    rec = {
        "value": cfg.seq_len / est,
        "unit": "tokens/s",
        "cores": int(blas["blas_threads"]),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle: {desc}; whole workload est. {est:.0f} s",
        "seconds_extrapolated": est,
        "seconds_measured": measured,
        "host_cpus": len(os.sched_getaffinity(0)),
        "blas": blas["blas"],
        "blas_threads": blas["blas_threads"],
    }
    rec["single_core"] = _single_core_oracle()
    return rec


def _time_call(fn, stream, reps):
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def without_lse_timing(cfg, shape, q, k, v, idx, out, ws, stream, t_attn, reps=5):
    """The attention call with lse_out = NULL (O only): the kernel variant without the
    float32 weight sum. The step above writes the LSE; this is the same call for a
    caller that does not need it."""
    from long_context_approximate_amd import spava
    ms = _time_call(lambda: spava.spava_approx_attn_fwd(shape, q, k, v, idx, out, None, ws, stream),
                    stream, reps)
    return {"attn_ms": ms, "tflops": attn_flops(cfg) / ms / 1e9,
            "speedup_vs_with_lse": t_attn * 1e3 / ms}


def time_schedules(cfg, q, k, v, idx, out, lse, ws, stream, reps=3):
    """Attention-call time under each dispatch order (the shape's schedule field; same
    results, different timing)."""
    from long_context_approximate_amd import spava
    res = {}
    for mode in ("lpt", "zigzag", "natural"):
        shape = spava.shape_from_config(cfg, schedule=spava.SCHEDULES[mode])
        res[mode] = _time_call(
            lambda: spava.spava_approx_attn_fwd(shape, q, k, v, idx, out, lse, ws, stream),
            stream, reps)
    return res


def dense_baseline(cfg, q, k, v, stream, t_step, reps=3):
    """Dense causal attention (one host: nothing passed, every key local) on the same
    inputs and the same kernel: the one-GPU analogue of the FlashAttention baseline."""
    import torch

    from long_context_approximate_amd import spava
    dense = cfg.with_(num_hosts=1, anchor_len=0, passing_len=0, window=1)
    shape = spava.shape_from_config(dense)
    out = torch.empty_like(q)
    ws = torch.empty(spava.spava_attn_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    idx = torch.empty((0, cfg.num_kv_heads, 0), dtype=torch.int32, device="cuda")
    ms = _time_call(lambda: spava.spava_approx_attn_fwd(shape, q, k, v, idx, out, None, ws, stream),
                    stream, reps)
    flops = attn_flops(dense)
    return {"attn_ms": ms, "tflops": flops / ms / 1e9, "flops": flops,
            "approx_step_speedup": ms / (t_step * 1e3)}


def query_block_timing(cfg, shape, k, v, stream, n_query=256, reps=5):
    """A 256-row query block after the context: its exact attention (H + 1 partials +
    log-sum-exp merge) and the query-aware passing selection, on this workload."""
    import torch

    from long_context_approximate_amd import spava
    from long_context_approximate_amd.inputs import make_inputs
    qcfg = cfg.with_(seq_len=n_query, num_hosts=1, anchor_len=0, window=1, seed=cfg.seed + 500)
    qd = spava.device_tensors(make_inputs(qcfg), "cuda:0")
    out = torch.empty_like(qd["q"])
    ws_q = torch.empty(spava.spava_query_workspace_bytes(shape, n_query), dtype=torch.uint8,
                       device="cuda")
    attn_ms = _time_call(lambda: spava.spava_query_attn_fwd(shape, qd["q"], qd["k"], qd["v"], k, v,
                                                            out, None, ws_q, stream), stream, reps)
    H, hkv, l = cfg.num_hosts, cfg.num_kv_heads, cfg.passing_len
    idx = torch.empty((max(H - 1, 0), hkv, l), dtype=torch.int32, device="cuda")
    ws_s = torch.empty(max(spava.spava_select_query_workspace_bytes(shape, n_query), 1),
                       dtype=torch.uint8, device="cuda")
    sel_ms = _time_call(lambda: spava.spava_select_passing_query(shape, qd["q"], k, idx, None,
                                                                 ws_s, stream), stream, reps)
    flops = 4.0 * cfg.head_dim * cfg.num_q_heads * n_query * (cfg.seq_len + (n_query + 1) / 2)
    return {"n_query": n_query, "attn_ms": attn_ms, "attn_tflops": flops / attn_ms / 1e9,
            "query_aware_select_ms": sel_ms}


def overlap_timing(shape, q, k, v, idx, out, lse, stream, t_step, reps=5):
    """The same layer through the overlapped entry: selection + passing gather on a
    side stream beside the passing-independent attention part (one-GPU form of the
    pages' overlapped transfers)."""
    import torch

    from long_context_approximate_amd import spava
    ws = torch.empty(spava.spava_layer_overlap_workspace_bytes(shape), dtype=torch.uint8,
                     device="cuda")
    side = torch.cuda.Stream()
    ms = _time_call(lambda: spava.spava_layer_overlap_fwd(shape, q, k, v, idx, out, lse, None, ws,
                                                          stream, side), stream, reps)
    return {"step_ms": ms, "serial_step_ms": t_step * 1e3, "speedup": t_step * 1e3 / ms}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="h8_128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the dense (one host) baseline, the schedule comparison, the "
                         "query block and the overlapped layer")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before warmup; its "
                         "FETCH_SIZE/WRITE_SIZE counters calibrate the HBM traffic figures")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the approximate-attention path runs all virtual hosts "
              "on a single MI355X (no multi-GPU mode). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_approximate_amd import spava
    from long_context_approximate_amd.inputs import CONFIGS, make_inputs

    cfg = CONFIGS[args.workload]
    torch.cuda.set_device(0)
    x = make_inputs(cfg)
    dev = spava.device_tensors(x, "cuda:0")
    q, k, v = dev["q"], dev["k"], dev["v"]
    shape = spava.shape_from_config(cfg)
    H, hkv, l, nb = cfg.num_hosts, cfg.num_kv_heads, cfg.passing_len, cfg.block_len
    idx = torch.empty((max(H - 1, 0), hkv, l), dtype=torch.int32, device="cuda")
    out = torch.empty((cfg.seq_len, cfg.num_q_heads, cfg.head_dim), dtype=q.dtype, device="cuda")
    lse = torch.empty((cfg.num_q_heads, cfg.seq_len), dtype=torch.float32, device="cuda")
    ws_sel = torch.empty(max(spava.spava_select_workspace_bytes(shape), 1), dtype=torch.uint8,
                         device="cuda")
    ws_attn = torch.empty(max(spava.spava_attn_workspace_bytes(shape), 1), dtype=torch.uint8,
                          device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        spava.spava_select_passing(shape, q, k, idx, None, ws_sel, stream)
        if ev is not None:
            ev[1].record(stream)
        spava.spava_approx_attn_fwd(shape, q, k, v, idx, out, lse, ws_attn, stream)
        if ev is not None:
            ev[2].record(stream)

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_sel = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps / 1e3
    t_attn = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps / 1e3
    t_step = wall / args.steps
    assert torch.isfinite(out.float()).all().item(), "non-finite output"

    flops = attn_flops(cfg)
    tflops = flops / t_attn / 1e12
    rec = {
        "metric": METRIC,
        "value": cfg.seq_len / t_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "seq_len": cfg.seq_len, "hosts": H,
                   "q_heads": cfg.num_q_heads, "kv_heads": hkv, "head_dim": cfg.head_dim,
                   "anchor": cfg.anchor_len, "passing": l, "window": cfg.window,
                   "keys": cfg.dist, "parallelism": "single GPU, all hosts in one grid"},
        "tflops": tflops,
        "frac_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "attn_tokens_per_s": cfg.seq_len / t_attn,
        "t_select_ms": t_sel * 1e3,
        "t_attn_ms": t_attn * 1e3,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic_from_profile(cfg.name)},
    }
    rec["score_fp64_gflops"] = score_flops(cfg) / t_sel / 1e9
    clock = clock_from_profile(cfg.name)
    clock_dur = _profile_field(cfg.name, "attn_clock_dur_us")
    if clock is not None and clock_dur:
        # The published peak assumes 2.4 GHz; under sustained matrix load the chip runs
        # slower (and the clock differs from box to box), so the counter run's own
        # kernel time is set against the peak at the clock measured in that run.
        adj = PEAK_BF16_TFLOPS * clock / PEAK_CLOCK_GHZ
        prof_tflops = flops / (clock_dur * 1e-6) / 1e12
        rec["clock_adjusted"] = {"clock_ghz": clock, "peak": adj, "tflops": prof_tflops,
                                 "frac": prof_tflops / adj}
    # From the committed counter runs of this attention source (None when stale):
    # matrix-core busy fraction and HBM rate of the attention kernel, and the gather
    # (prep) kernel's duration.
    busy = _profile_field(cfg.name, "attn_mfma_busy_frac")
    dur = _profile_field(cfg.name, "attn_kernel", "dur_us")
    hbm = traffic_from_profile(cfg.name)
    rec["profiled"] = {
        "attn_mfma_busy_frac": busy,
        "attn_hbm_gb_per_s": hbm / dur / 1e3 if hbm is not None and dur else None,
        "t_gather_ms": (lambda v: v / 1e3 if v is not None else None)(
            _profile_field(cfg.name, "prep_kernel", "dur_us")),
    }
    if not args.no_extras:
        rec["schedules_attn_ms"] = time_schedules(cfg, q, k, v, idx, out, lse, ws_attn, stream)
        rec["attn_without_lse"] = without_lse_timing(cfg, shape, q, k, v, idx, out, ws_attn,
                                                     stream, t_attn)
        rec["dense_causal"] = dense_baseline(cfg, q, k, v, stream, t_step)
        rec["query_block"] = query_block_timing(cfg, shape, k, v, stream)
        rec["overlap"] = overlap_timing(shape, q, k, v, idx, out, lse, stream, t_step)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, x)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
