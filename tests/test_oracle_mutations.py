"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutation is a plausible slip in the oracle's arithmetic or bookkeeping. The test
swaps it into the oracle module with monkeypatch, runs the pins that should catch
it, and requires an AssertionError. This shows the pins are sharp enough to notice
a dropped term, a wrong index, an off-by-one mask or a reversed tie rule.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.spava_oracle as so
import tests.test_oracle_pins as pins


def _attention_rows_exclusive_diagonal(sh, q, k, v, idx, hq, rows):
    rows = np.asarray(rows, dtype=np.int64)
    g = hq // sh.group
    h = int(rows[0] // sh.block_len)
    s, e = so.context_block(sh, h)
    pre = so.visible_prefix(sh, idx, h, g)
    local = np.arange(s, e, dtype=np.int64)
    keys = np.concatenate([pre, local])
    x = sh.scale * (q[rows, hq, :] @ k[keys, g, :].T)
    hidden = np.zeros(x.shape, dtype=bool)
    hidden[:, len(pre):] = local[None, :] >= rows[:, None]   # slip: own key hidden
    hidden[:, len(pre)] &= local[0] != rows                 # keep row s_h non-empty
    x = np.where(hidden, -np.inf, x)
    m = x.max(axis=1, keepdims=True)
    ex = np.exp(x - m)
    z = ex.sum(axis=1, keepdims=True)
    return (ex / z) @ v[keys, g, :], m[:, 0] + np.log(z[:, 0])


def _visible_prefix_without_anchor(sh, idx, h, g):
    if h == 0:
        return np.zeros(0, dtype=np.int64)
    parts = [np.zeros(0, dtype=np.int64)]                   # slip: anchor dropped
    for j in range(h):
        sel = idx[j, g]
        parts.append(sel[sel >= 0].astype(np.int64))
    return np.concatenate(parts)


def _select_ties_to_higher(sh, scores):
    H, hkv, l = sh.num_hosts, sh.num_kv_heads, sh.passing_len
    idx = np.full((max(H - 1, 0), hkv, l), -1, dtype=np.int32)
    for j in range(H - 1):
        s, _ = so.context_block(sh, j)
        cand = so.passing_candidates(sh, j)
        lj = so.passing_length(sh, j)
        for g in range(hkv):
            sc = scores[j, g, cand - s]
            order = np.lexsort((-cand, -sc))                # slip: ties to higher position
            idx[j, g, :lj] = np.sort(cand[order[:lj]])
    return idx


def _window_scores_noncausal(sh, q, k, j, g):
    s, e = so.context_block(sh, j)
    G, w = sh.group, sh.window
    kl = k[s:e, g, :]
    total = np.zeros(e - s)
    for hq in range(g * G, (g + 1) * G):
        x = sh.scale * (q[e - w:e, hq, :] @ kl.T)          # slip: no causal mask
        ex = np.exp(x - x.max(axis=1, keepdims=True))
        total += (ex / ex.sum(axis=1, keepdims=True)).sum(axis=0)
    return total / (G * w)


def _window_scores_unscaled(sh, q, k, j, g):
    s, e = so.context_block(sh, j)
    G, w = sh.group, sh.window
    obs = np.arange(e - w, e)
    keys = np.arange(s, e)
    total = np.zeros(e - s)
    for hq in range(g * G, (g + 1) * G):
        x = q[e - w:e, hq, :] @ k[s:e, g, :].T               # slip: scale dropped
        x = np.where(keys[None, :] <= obs[:, None], x, -np.inf)
        ex = np.exp(x - x.max(axis=1, keepdims=True))
        total += (ex / ex.sum(axis=1, keepdims=True)).sum(axis=0)
    return total / (G * w)


def _candidates_with_anchor(sh, j):
    s, e = so.context_block(sh, j)
    return np.arange(s, e, dtype=np.int64)                  # slip: anchor passable


MUTATIONS = [
    ("attention_rows", _attention_rows_exclusive_diagonal,
     [lambda: pins.test_one_host_is_dense_causal_attention(16)]),
    ("visible_prefix", _visible_prefix_without_anchor,
     [pins.test_anchor_only_matches_explicit_mask]),
    ("select_passing", _select_ties_to_higher,
     [pins.test_zero_queries_closed_form]),
    ("window_scores", _window_scores_noncausal,
     [lambda: pins.test_tiny_bruteforce_selection_and_attention(1)]),
    ("window_scores", _window_scores_unscaled,
     [lambda: pins.test_tiny_bruteforce_selection_and_attention(2)]),
    ("passing_candidates", _candidates_with_anchor,
     [lambda: pins.test_passing_everything_is_dense_causal_attention(2, 5, 64)]),
]


@pytest.mark.parametrize("name,bad,checks", MUTATIONS,
                         ids=[m[1].__name__.strip("_") for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, bad, checks):
    monkeypatch.setattr(so, name, bad)          # calls inside the module
    monkeypatch.setattr(oracle, name, bad)      # calls through the package
    for check in checks:
        with pytest.raises(AssertionError):
            check()
