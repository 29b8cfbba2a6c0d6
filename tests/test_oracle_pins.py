"""Pins for the fp64 oracle, against facts fixed outside the oracle itself.

Each test ties one part of the oracle to something independent of its code:
  * a library routine (torch scaled_dot_product_attention, float64 on the CPU) for the
    cases where the method reduces to dense or block-diagonal causal attention: one
    host (the explainer's "Einschraenkungen": on a single GPU the method is standard
    FlashAttention), or every earlier row passed;
  * closed forms (all-zero queries);
  * brute force on tiny inputs: 40-digit Decimal scores and a position-by-position
    visibility predicate, a different formulation from the oracle's segment lists;
  * exact rational arithmetic (w = 1, G = 1 reduces selection to exact dot products);
  * invariants (probability mass sums to one, visible-set sizes).
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc

RNG = np.random.default_rng(12345)


def _bf16_exact(shape, rng=RNG, scale=1.0):
    """float64 arrays holding bf16-representable values (as the stored inputs are)."""
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    u = x.view(np.uint32)
    u = ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    return orc.bf16_bits_to_f64(u)


def _qkv(sh, rng=RNG):
    n, hq, hkv, d = sh.seq_len, sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    return (_bf16_exact((n, hq, d), rng), _bf16_exact((n, hkv, d), rng),
            _bf16_exact((n, hkv, d), rng))


def _sdpa(q, k, v, sh, mask=None, causal=False):
    """torch SDPA in float64; q [N,Hq,d], k/v [N,Hkv,d]; GQA head hq -> hq // G."""
    G = sh.group
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, is_causal=causal, scale=sh.scale)
    return o[0].permute(1, 0, 2).numpy()


def _causal_lse(q, k, sh, allowed):
    """torch.logsumexp of the logits over an explicit boolean [N, N] visibility matrix."""
    G = sh.group
    out = np.zeros((sh.num_q_heads, sh.seq_len))
    for hq in range(sh.num_q_heads):
        x = torch.from_numpy(q[:, hq, :]) @ torch.from_numpy(k[:, hq // G, :]).T * sh.scale
        x = x.masked_fill(~torch.from_numpy(allowed), float("-inf"))
        out[hq] = torch.logsumexp(x, dim=1).numpy()
    return out


# ------------------------------------------------------------------ library pins

@pytest.mark.parametrize("d", [16, 64])
def test_one_host_is_dense_causal_attention(d):
    sh = orc.Shape(96, 1, 4, 2, d, 0, 8, 5)
    q, k, v = _qkv(sh)
    idx = orc.select_passing(sh, orc.all_window_scores(sh, q, k))
    assert idx.shape == (0, 2, 8)
    o, lse = orc.approx_attention(sh, q, k, v, idx)
    ref = _sdpa(q, k, v, sh, causal=True)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    tri = np.tril(np.ones((96, 96), dtype=bool))
    np.testing.assert_allclose(lse, _causal_lse(q, k, sh, tri), rtol=0, atol=1e-12)


@pytest.mark.parametrize("H,A,l", [(2, 5, 64), (3, 0, 40), (4, 8, 1000), (4, 24, 24)])
def test_passing_everything_is_dense_causal_attention(H, A, l):
    # With l >= |C_j| every earlier row is passed, so each query sees its whole
    # causal prefix exactly once: the result is dense causal attention.
    sh = orc.Shape(24 * H, H, 6, 2, 16, A, l, 7)
    q, k, v = _qkv(sh)
    idx = orc.select_passing(sh, orc.all_window_scores(sh, q, k))
    o, lse = orc.approx_attention(sh, q, k, v, idx)
    np.testing.assert_allclose(o, _sdpa(q, k, v, sh, causal=True), rtol=0, atol=1e-12)
    tri = np.tril(np.ones((sh.seq_len, sh.seq_len), dtype=bool))
    np.testing.assert_allclose(lse, _causal_lse(q, k, sh, tri), rtol=0, atol=1e-12)


def test_no_anchor_no_passing_is_block_diagonal_causal():
    sh = orc.Shape(60, 3, 4, 4, 16, 0, 0, 4)
    q, k, v = _qkv(sh)
    idx = orc.select_passing(sh, orc.all_window_scores(sh, q, k))
    assert idx.size == 0 or np.all(idx == -1)
    o, _ = orc.approx_attention(sh, q, k, v, idx)
    for h in range(3):
        s, e = orc.context_block(sh, h)
        ref = _sdpa(q[s:e], k[s:e], v[s:e], sh, causal=True)
        np.testing.assert_allclose(o[s:e], ref, rtol=0, atol=1e-12)


def test_anchor_only_matches_explicit_mask():
    # l = 0: blocks h >= 1 see the anchor and their own causal prefix.
    sh = orc.Shape(48, 3, 2, 1, 16, 5, 0, 4)
    q, k, v = _qkv(sh)
    idx = orc.select_passing(sh, orc.all_window_scores(sh, q, k))
    o, lse = orc.approx_attention(sh, q, k, v, idx)
    n, nb = sh.seq_len, sh.block_len
    allowed = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for p in range(n):
            same = p // nb == i // nb and p <= i
            anchor = p < sh.anchor_len and i // nb >= 1
            allowed[i, p] = same or anchor
    ref = _sdpa(q, k, v, sh, mask=torch.from_numpy(allowed))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _causal_lse(q, k, sh, allowed), rtol=0, atol=1e-12)


# ------------------------------------------------------------------- closed forms

def test_zero_queries_closed_form():
    # q = 0: every logit is 0, so O is the plain mean of the visible values,
    # LSE = log |V(i)|, and every key a whole window sees ties exactly, so the tie
    # rule picks the lowest candidate positions.
    sh = orc.Shape(64, 4, 4, 2, 16, 3, 5, 4)
    _, k, v = _qkv(sh)
    q = np.zeros((sh.seq_len, sh.num_q_heads, sh.head_dim))
    scores = orc.all_window_scores(sh, q, k)
    idx = orc.select_passing(sh, scores)
    for j in range(sh.num_hosts - 1):
        cand = orc.passing_candidates(sh, j)
        for g in range(sh.num_kv_heads):
            assert list(idx[j, g]) == list(cand[:sh.passing_len])
            # closed-form score for a key every observer sees:
            s, e = orc.context_block(sh, j)
            expect = sum(1.0 / (i - s + 1) for i in range(e - sh.window, e)) / sh.window
            assert scores[j, g, 0] == pytest.approx(expect, rel=1e-15)
    o, lse = orc.approx_attention(sh, q, k, v, idx)
    G = sh.group
    for i in range(sh.seq_len):
        h = i // sh.block_len
        s, _ = orc.context_block(sh, h)
        for hq in range(sh.num_q_heads):
            g = hq // G
            vis = list(range(sh.anchor_len)) if h else []
            for j in range(h):
                vis += [p for p in idx[j, g] if p >= 0]
            vis += list(range(s, i + 1))
            np.testing.assert_allclose(o[i, hq], v[vis, g].mean(axis=0), rtol=0, atol=1e-13)
            assert lse[hq, i] == pytest.approx(math.log(len(vis)), abs=1e-13)


# ------------------------------------------------------------- tiny brute force

def _decimal_scores(sh, q, k, j, g):
    getcontext().prec = 40
    s, e = orc.context_block(sh, j)
    scale = Decimal(sh.scale)
    total = [Decimal(0)] * (e - s)
    for hq in range(g * sh.group, (g + 1) * sh.group):
        for i in range(e - sh.window, e):
            xs = [scale * sum(Decimal(float(a)) * Decimal(float(b))
                              for a, b in zip(q[i, hq], k[p, g])) for p in range(s, i + 1)]
            m = max(xs)
            ex = [(x - m).exp() for x in xs]
            z = sum(ex)
            for t, val in enumerate(ex):
                total[t] += val / z
    return [t / (sh.group * sh.window) for t in total]


def _brute_selection(sh, q, k):
    sel = {}
    for j in range(sh.num_hosts - 1):
        s, e = orc.context_block(sh, j)
        for g in range(sh.num_kv_heads):
            sc = _decimal_scores(sh, q, k, j, g)
            lo = max(s, sh.anchor_len) if j == 0 else s
            cand = sorted(range(lo, e), key=lambda p: (-sc[p - s], p))
            sel[(j, g)] = set(cand[:sh.passing_len])
    return sel


def _brute_attention(sh, q, k, v, sel):
    """Pure-Python attention from a per-position visibility predicate."""
    n, nb, G = sh.seq_len, sh.block_len, sh.group
    o = np.zeros((n, sh.num_q_heads, sh.head_dim))
    lse = np.zeros((sh.num_q_heads, n))

    def visible(p, i, g):
        hp, hi = p // nb, i // nb
        if hp == hi:
            return p <= i
        if hp > hi:
            return False
        if p < sh.anchor_len:
            return True
        return p in sel[(hp, g)]

    for i in range(n):
        for hq in range(sh.num_q_heads):
            g = hq // G
            vis = [p for p in range(n) if visible(p, i, g)]
            xs = [sh.scale * math.fsum(float(a) * float(b) for a, b in zip(q[i, hq], k[p, g]))
                  for p in vis]
            m = max(xs)
            ex = [math.exp(x - m) for x in xs]
            z = math.fsum(ex)
            for t in range(sh.head_dim):
                o[i, hq, t] = math.fsum(e_ * v[p, g, t] for e_, p in zip(ex, vis)) / z
            lse[hq, i] = m + math.log(z)
    return o, lse


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_tiny_bruteforce_selection_and_attention(seed):
    rng = np.random.default_rng(seed)
    sh = orc.Shape(24, 3, 4, 2, 8, 2, 3, 3)
    q, k, v = _qkv(sh, rng)
    scores = orc.all_window_scores(sh, q, k)
    for j in range(sh.num_hosts - 1):
        for g in range(sh.num_kv_heads):
            dec = _decimal_scores(sh, q, k, j, g)
            np.testing.assert_allclose(scores[j, g], [float(x) for x in dec], rtol=1e-13, atol=0)
    idx = orc.select_passing(sh, scores)
    sel = _brute_selection(sh, q, k)
    for (j, g), chosen in sel.items():
        got = [int(p) for p in idx[j, g] if p >= 0]
        assert got == sorted(chosen)
    o, lse = orc.approx_attention(sh, q, k, v, idx)
    bo, blse = _brute_attention(sh, q, k, v, sel)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


def test_window_one_group_one_is_exact_dot_product_ranking():
    # w = 1, G = 1: one observer; exp is monotone, so the ranking is that of the exact
    # (rational) dot products of the observer with every candidate key.
    rng = np.random.default_rng(7)
    sh = orc.Shape(120, 3, 2, 2, 16, 6, 9, 1)
    q, k, _ = _qkv(sh, rng)
    idx = orc.select_passing(sh, orc.all_window_scores(sh, q, k))
    for j in range(2):
        s, e = orc.context_block(sh, j)
        lo = max(s, sh.anchor_len) if j == 0 else s
        for g in range(2):
            dots = {p: sum(Fraction(float(a)) * Fraction(float(b))
                           for a, b in zip(q[e - 1, g], k[p, g])) for p in range(lo, e)}
            best = sorted(dots, key=lambda p: (-dots[p], p))[:sh.passing_len]
            assert [int(p) for p in idx[j, g]] == sorted(best)


def test_duplicated_keys_tie_to_lower_position():
    rng = np.random.default_rng(11)
    sh = orc.Shape(96, 3, 2, 1, 16, 4, 6, 4)
    q, k, _ = _qkv(sh, rng)
    # Block 1 is [32, 64); its window is queries 60..63 of both heads. Give every
    # observer the same query u and copy one key 2u to positions 40, 45 and 50: the
    # three keys then score exactly alike and above every other key.
    u = q[0, 0].copy()
    q[60:64, :, :] = u
    k[40, 0] = 2.0 * u
    k[45, 0] = k[40, 0]
    k[50, 0] = k[40, 0]
    sh1 = orc.Shape(96, 3, 2, 1, 16, 4, 2, 4)   # pass only two rows
    scores = orc.all_window_scores(sh1, q, k)
    assert scores[1, 0, 40 - 32] == scores[1, 0, 45 - 32] == scores[1, 0, 50 - 32]
    idx = orc.select_passing(sh1, scores)
    assert list(idx[1, 0]) == [40, 45]


# ------------------------------------------------------------------- invariants

def test_invariants_scores_sum_to_one_and_visible_counts():
    rng = np.random.default_rng(5)
    sh = orc.Shape(200, 4, 6, 3, 16, 7, 11, 9)
    q, k, _ = _qkv(sh, rng)
    scores = orc.all_window_scores(sh, q, k)
    np.testing.assert_allclose(scores.sum(axis=2), 1.0, rtol=0, atol=1e-13)
    assert np.all(scores >= 0)
    idx = orc.select_passing(sh, scores)
    for j in range(sh.num_hosts - 1):
        s, e = orc.context_block(sh, j)
        for g in range(sh.num_kv_heads):
            sel = idx[j, g]
            assert np.all(np.diff(sel) > 0)                 # ascending, unique
            assert np.all((sel >= s) & (sel < e))
            if j == 0:
                assert np.all(sel >= sh.anchor_len)         # anchor never passed twice
    for i in [0, 49, 50, 77, 199]:
        h = i // sh.block_len
        for g in range(sh.num_kv_heads):
            pre = orc.visible_prefix(sh, idx, h, g)
            assert len(set(pre.tolist())) == len(pre)       # disjoint parts
            expect = (sh.anchor_len + sh.passing_len * h if h else 0) + i - h * 50 + 1
            assert orc.visible_count(sh, idx, i, g) == expect


def test_passing_lengths_clip_to_candidates():
    sh = orc.Shape(40, 4, 1, 1, 8, 6, 7, 2)
    assert [orc.passing_length(sh, j) for j in range(3)] == [4, 7, 7]
    sh = orc.Shape(40, 4, 1, 1, 8, 10, 7, 2)
    assert orc.passing_length(sh, 0) == 0
    rng = np.random.default_rng(3)
    q, k, _ = _qkv(sh, rng)
    idx = orc.select_passing(sh, orc.all_window_scores(sh, q, k))
    assert np.all(idx[0] == -1)


def test_query_block_is_the_tail_of_dense_causal_attention():
    # B_qr appended after the context: its rows of a dense causal attention over
    # [context ; query] see every context key and the earlier query keys (library pin).
    rng = np.random.default_rng(31)
    sh = orc.Shape(60, 3, 4, 2, 16, 4, 5, 3)
    q, k, v = _qkv(sh, rng)
    nq = 9
    q_qr, k_qr, v_qr = (_bf16_exact((nq, 4, 16), rng), _bf16_exact((nq, 2, 16), rng),
                        _bf16_exact((nq, 2, 16), rng))
    o, lse = orc.query_block_attention(sh, q_qr, k_qr, v_qr, k, v)
    cat = orc.Shape(60 + nq, 1, 4, 2, 16, 0, 0, 1)
    qc = np.concatenate([q, q_qr]); kc = np.concatenate([k, k_qr]); vc = np.concatenate([v, v_qr])
    ref = _sdpa(qc, kc, vc, cat, causal=True)[60:]
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    tri = np.tril(np.ones((60 + nq, 60 + nq), dtype=bool))
    np.testing.assert_allclose(lse, _causal_lse(qc, kc, cat, tri)[:, 60:], rtol=0, atol=1e-12)


def test_query_aware_scores_decimal_bruteforce_and_invariants():
    rng = np.random.default_rng(33)
    sh = orc.Shape(24, 3, 4, 2, 8, 2, 3, 3)
    _, k, _ = _qkv(sh, rng)
    q_qr = _bf16_exact((5, 4, 8), rng)
    getcontext().prec = 40
    scores = orc.all_query_scores(sh, q_qr, k)
    np.testing.assert_allclose(scores.sum(axis=2), 1.0, rtol=0, atol=1e-14)
    for j in range(2):
        s, e = orc.context_block(sh, j)
        for g in range(2):
            total = [Decimal(0)] * (e - s)
            for hq in range(2 * g, 2 * g + 2):
                for i in range(5):
                    xs = [Decimal(sh.scale) * sum(Decimal(float(a)) * Decimal(float(b))
                                                  for a, b in zip(q_qr[i, hq], k[p, g]))
                          for p in range(s, e)]
                    m = max(xs)
                    ex = [(x - m).exp() for x in xs]
                    z = sum(ex)
                    for t, val in enumerate(ex):
                        total[t] += val / z
            ref = [float(t / 10) for t in total]
            np.testing.assert_allclose(scores[j, g], ref, rtol=1e-13, atol=0)


def test_query_aware_scores_equal_window_scores_of_a_last_row_observer():
    # One observer equal to block j's last query sees every key of the block under the
    # causal rule too, so the two scorings coincide (w = 1, G = 1).
    rng = np.random.default_rng(34)
    sh = orc.Shape(64, 2, 2, 2, 16, 3, 5, 1)
    q, k, _ = _qkv(sh, rng)
    win = orc.all_window_scores(sh, q, k)
    q_qr = q[31:32].copy()                     # block 0 ends at 32
    qa = orc.all_query_scores(sh, q_qr, k)
    np.testing.assert_allclose(qa, win, rtol=1e-15, atol=0)


# ------------------------------------------------------ input widening and margins

def _bf16_value_from_definition(bits: int) -> float:
    """Value of a bf16 bit pattern from the format's definition: 1 sign bit, 8 exponent
    bits (bias 127), 7 fraction bits; exponent 0 is subnormal (2^-126 * f/128),
    exponent 255 is infinity (f == 0) or NaN."""
    sign = -1.0 if bits >> 15 else 1.0
    e, f = (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0xFF:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


def test_bf16_widening_on_every_bit_pattern():
    # All 65536 patterns: the oracle's widening must give the value torch's own bfloat16
    # -> float64 conversion gives, and the value the format's definition gives, bit for
    # bit (signed zeros, subnormals and infinities included; NaN stays NaN).
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_bits_to_f64(bits)
    via_to_f64 = orc.to_f64(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    defn = np.array([_bf16_value_from_definition(int(b)) for b in bits])
    for name, ref in (("torch", lib), ("definition", defn)):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), name
        assert np.array_equal(got[~nan].view(np.uint64), ref[~nan].view(np.uint64)), name
    assert np.array_equal(via_to_f64.view(np.uint64), got.view(np.uint64))
    assert got.dtype == np.float64 and via_to_f64.dtype == np.float64


def _margin_fraction(sh, scores, j, g):
    """Relative gap between the l_j-th and (l_j + 1)-th largest candidate scores of
    block j, in exact rational arithmetic; None when nothing is selected or nothing is
    rejected. Candidates are listed from the definition: block j's positions, minus the
    anchor [0, A) for block 0."""
    nb, A, l = sh.block_len, sh.anchor_len, sh.passing_len
    cand = [p for p in range(j * nb, (j + 1) * nb) if not (j == 0 and p < A)]
    lj = min(l, len(cand))
    if lj == 0 or lj == len(cand):
        return None
    vals = sorted((Fraction(float(scores[j, g, p - j * nb])) for p in cand), reverse=True)
    return (vals[lj - 1] - vals[lj]) / vals[lj - 1]


def test_selection_margins_worked_example():
    # N = 12, H = 3 (blocks of 4), A = 2, l = 2, two KV heads. Block 0's candidates are
    # positions 2, 3 only (the anchor is excluded), so l_0 = |C_0| and nothing is
    # rejected: NaN. Block 1, head 0: scores 1/2, 1/8, 1/4, 1/8 -> sorted 1/2, 1/4,
    # 1/8, 1/8; the 2nd (1/4) against the 3rd (1/8): (1/4 - 1/8) / (1/4) = 1/2.
    # Block 1, head 1: a tie at the boundary (3/8, 1/8, 1/8, 1/8 -> 1/8 vs 1/8) gives 0.
    # The anchor rows of block 0 carry a huge score that must not count.
    sh = orc.Shape(12, 3, 2, 2, 4, 2, 2, 1)
    scores = np.zeros((2, 2, 4))
    scores[0, :, :] = [1e9, 1e9, 0.25, 0.75]
    scores[1, 0, :] = [0.5, 0.125, 0.25, 0.125]
    scores[1, 1, :] = [0.375, 0.125, 0.125, 0.125]
    m = orc.selection_margins(sh, scores)
    assert m.shape == (2, 2)
    assert np.isnan(m[0]).all()
    assert m[1, 0] == 0.5
    assert m[1, 1] == 0.0
    # l = 0: nothing is selected anywhere.
    assert np.isnan(orc.selection_margins(orc.Shape(12, 3, 2, 2, 4, 2, 0, 1), scores)).all()
    # One host: no block passes rows, so there is nothing to report.
    assert orc.selection_margins(orc.Shape(4, 1, 2, 2, 4, 0, 2, 1), np.zeros((0, 2, 4))).shape \
        == (0, 2)


@pytest.mark.parametrize("A,l", [(0, 3), (5, 3), (5, 11), (3, 16), (0, 16), (7, 1)])
def test_selection_margins_match_exact_rationals(A, l):
    # Random positive scores (with repeated values, so ties occur), checked against the
    # exact rational gap of the definition; NaN exactly where nothing is rejected.
    rng = np.random.default_rng(100 + 7 * A + l)
    sh = orc.Shape(48, 3, 4, 2, 8, A, l, 2)
    scores = rng.choice(rng.random(9) + 0.01, size=(2, 2, 16))
    m = orc.selection_margins(sh, scores)
    for j in range(2):
        for g in range(2):
            ref = _margin_fraction(sh, scores, j, g)
            if ref is None:
                assert np.isnan(m[j, g]), (j, g)
            else:
                assert abs(Fraction(float(m[j, g])) - ref) <= abs(ref) * Fraction(1, 2 ** 50), \
                    (j, g, float(m[j, g]), float(ref))
