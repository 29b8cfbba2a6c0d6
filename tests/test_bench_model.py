"""Host checks of the benchmark's work model and JSON contract pieces (no GPU).

The key-visit count behind the reported TFLOP/s is compared with an independent
brute-force count of visible (query, key) pairs on small shapes, and its closed form
with hand-computed values for the named workloads.
"""
from __future__ import annotations

import numpy as np
import pytest

import bench
import oracle
from long_context_approximate_amd.inputs import CONFIGS, small_config


def _brute_force_visits(cfg):
    """Count every query's visible keys with the oracle's own visibility rule, under a
    valid selection (equal scores: the lowest candidates)."""
    sh = oracle.shape_of(cfg)
    H, hkv, nb = cfg.num_hosts, cfg.num_kv_heads, cfg.block_len
    idx = oracle.select_passing(sh, np.zeros((max(H - 1, 0), hkv, nb)))
    return sum(oracle.visible_count(sh, idx, i, 0) for i in range(cfg.seq_len))


@pytest.mark.parametrize("cfg", [
    small_config(),
    small_config(name="bm1", seq_len=1024, num_hosts=4, anchor_len=40, passing_len=300),
    small_config(name="bm2", seq_len=1000, num_hosts=1, anchor_len=0),
    small_config(name="bm3", seq_len=1536, num_hosts=3, anchor_len=0, passing_len=0),
    CONFIGS["tiny_f32_512"],
], ids=lambda c: c.name)
def test_key_visits_match_brute_force(cfg):
    assert bench.key_visits_per_head(cfg) == _brute_force_visits(cfg)


# Per-head key visits sum_h [n_b(n_b+1)/2 + [h>=1] n_b (A + P_h)], worked by hand:
#   16K:  4 x 4096*4097/2 + 4096*(1024*3 + 512*(1+2+3))
#         = 33,562,624 + 25,165,824 = 58,728,448
#   128K: 8 x 16384*16385/2 + 16384*(4096*7 + 2048*(1+...+7))
#         = 1,073,807,360 + 1,409,286,144 = 2,483,093,504
@pytest.mark.parametrize("name,visits", [
    ("tiny_f32_512", 78_080),
    ("h4_16k", 58_728_448),
    ("video_h8_64k", 620_789_760),
    ("h8_128k", 2_483_093_504),
    ("t3_h16_256k", 7_180_779_520),
])
def test_key_visits_named_workloads(name, visits):
    assert bench.key_visits_per_head(CONFIGS[name]) == visits


def test_attention_flops_128k():
    cfg = CONFIGS["h8_128k"]
    assert bench.attn_flops(cfg) == pytest.approx(4 * 128 * 28 * 2_483_093_504)
    assert bench.attn_flops(cfg) == pytest.approx(3.56e13, rel=2e-3)


def test_gpus_above_one_exit_with_a_message(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def _brute_force_score_visits(cfg):
    """Visible (observer row, key) pairs of the window scores, counted one by one: row i
    of the last w queries of block j >= 1 sees the block's keys up to i."""
    H, nb, w = cfg.num_hosts, cfg.block_len, cfg.window
    per_head = sum(i - j * nb + 1 for j in range(1, H) for i in range((j + 1) * nb - w, (j + 1) * nb))
    return per_head * cfg.num_q_heads   # G rows per KV head and Hkv KV heads = Hq rows


@pytest.mark.parametrize("cfg", [small_config(), CONFIGS["tiny_f32_512"], CONFIGS["h4_16k"]],
                         ids=lambda c: c.name)
def test_score_flops_match_brute_force(cfg):
    assert bench.score_flops(cfg) == 2 * cfg.head_dim * _brute_force_score_visits(cfg)


def test_score_flops_of_the_named_workloads():
    # 2 d (H-1) Hkv G (w n_b - w(w-1)/2), worked by hand for 128K:
    # 2*128 * 7*4*7 * (128*16384 - 8128) = 50,176 * 2,089,024 = 104,818,868,224
    assert bench.score_flops(CONFIGS["h8_128k"]) == 104_818_868_224
