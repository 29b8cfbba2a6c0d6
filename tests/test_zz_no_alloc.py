"""The allocation-free selection (spava_select_passing_noalloc) against the selection
that takes a workspace, through the C ABI, on two calls in a row: the second with a
smaller input, so it runs over scratch the first call left behind."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from long_context_approximate_amd.inputs import CONFIGS, make_inputs, small_config

pytestmark = pytest.mark.gpu


def _select(cfg, x, noalloc, with_scores=True):
    import torch
    from long_context_approximate_amd import spava
    dev = spava.device_tensors({"q": x["q"], "k": x["k"]}, "cuda")
    shape = spava.shape_from_config(cfg)
    H, hkv, l, nb = cfg.num_hosts, cfg.num_kv_heads, cfg.passing_len, cfg.block_len
    idx = torch.full((max(H - 1, 0), hkv, l), -7, dtype=torch.int32, device="cuda")
    sc = (torch.full((max(H - 1, 0), hkv, nb), -1.0, dtype=torch.float64, device="cuda")
          if with_scores else None)
    if noalloc:
        spava.spava_select_passing_noalloc(shape, dev["q"], dev["k"], idx, sc)
    else:
        spava.spava_select_passing(shape, dev["q"], dev["k"], idx, sc)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (sc.cpu().numpy() if sc is not None else None)


def _compare(cfg, x, with_scores=True):
    ref_idx, ref_sc = _select(cfg, x, noalloc=False)
    idx, sc = _select(cfg, x, noalloc=True, with_scores=with_scores)
    assert np.array_equal(idx, ref_idx), "indices differ from spava_select_passing"
    if with_scores:
        assert np.array_equal(sc.view(np.uint64), ref_sc.view(np.uint64)), \
            "scores differ from spava_select_passing"
    return ref_idx, ref_sc


def test_two_calls_in_a_row_second_smaller():
    big = small_config(name="na_big", seq_len=4096, num_hosts=4, num_q_heads=8, num_kv_heads=2,
                       anchor_len=100, passing_len=150, window=96, dist="student_t3", seed=81)
    small = small_config(name="na_small", seq_len=1500, num_hosts=3, num_q_heads=4,
                         num_kv_heads=2, anchor_len=30, passing_len=40, window=20, seed=82)
    for cfg in (big, small):
        x = make_inputs(cfg)
        idx, _ = _compare(cfg, x)
        ref = oracle.run(oracle.shape_of(cfg), x["q"], x["k"], x["v"], attention=False)
        assert np.array_equal(idx, ref["idx"])


def test_without_scores_out_the_scores_live_in_the_scratch():
    cfg = small_config(name="na_noscores", seq_len=3000, num_hosts=3, seed=83)
    x = make_inputs(cfg)
    _compare(cfg, x, with_scores=False)
    smaller = cfg.with_(name="na_noscores_small", seq_len=1200, num_hosts=2, seed=84)
    _compare(smaller, make_inputs(smaller), with_scores=False)


def test_full_size_128k_then_16k():
    # The 128K workload (7.3 MiB of scratch), then the 16K one over what it left.
    for name in ("h8_128k", "h4_16k"):
        cfg = CONFIGS[name]
        _compare(cfg, make_inputs(cfg))


def test_float32_and_d64_shapes():
    # The float32 selection kernels and head dimension 64 through the same scratch.
    for cfg in (small_config(name="na_f32", dtype="f32", seq_len=1200, num_hosts=4, seed=85),
                small_config(name="na_d64", head_dim=64, seq_len=2048, num_hosts=4,
                             num_q_heads=8, num_kv_heads=2, anchor_len=64, passing_len=128,
                             window=64, seed=86)):
        x = make_inputs(cfg)
        idx, _ = _compare(cfg, x)
        ref = oracle.run(oracle.shape_of(cfg), x["q"], x["k"], x["v"], attention=False)
        assert np.array_equal(idx, ref["idx"])


def test_captured_in_a_hip_graph_and_replayed():
    # The reason for the entry: it can be captured (nothing is allocated). Every replay,
    # with eager work and synchronisation in between, must give the eager result.
    import torch
    from long_context_approximate_amd import spava
    cfg = small_config(name="na_graph", seq_len=3000, num_hosts=3, seed=87)
    x = make_inputs(cfg)
    dev = spava.device_tensors({"q": x["q"], "k": x["k"]}, "cuda")
    shape = spava.shape_from_config(cfg)
    H, hkv, l, nb = cfg.num_hosts, cfg.num_kv_heads, cfg.passing_len, cfg.block_len
    idx = torch.empty((H - 1, hkv, l), dtype=torch.int32, device="cuda")
    sc = torch.empty((H - 1, hkv, nb), dtype=torch.float64, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        spava.spava_select_passing_noalloc(shape, dev["q"], dev["k"], idx, sc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = (idx.clone(), sc.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        spava.spava_select_passing_noalloc(shape, dev["q"], dev["k"], idx, sc)
    for rep in range(3):
        idx.zero_()
        sc.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(sc, ref[1]), f"replay {rep} differs"
    r = oracle.run(oracle.shape_of(cfg), x["q"], x["k"], x["v"], attention=False)
    assert np.array_equal(idx.cpu().numpy(), r["idx"])
