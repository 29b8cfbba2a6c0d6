"""Plain fp64 CPU oracle for Spava / APB-V prefill approximate attention.

TEST INFRASTRUCTURE ONLY. This package exists to check the HIP path. Only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may import it; the
library in ``long_context_approximate_amd`` never imports or calls it, and this
package imports nothing from that library.

Sources (pages about arXiv 2601.21444; cited by page title and section):
  [ABS]  "Spava: Accelerating Long-Video Understanding via Sequence-Parallelism-aware
         Approximate Attention", English abstract (shd-paper.top, fugumt.com) and the
         same abstract under the title "APB-V: ..." (info.umar.mx record).
  [METH] "APB-V: Accelerating Long-Video Understanding via Sequence-Parallelism-aware
         Approximate Attention" (gist.science explainer, German), Technisches
         Resuemee > "Methodik: APB-V" > 1. Framework-Design: Kontext-Splitting &
         ZigZag-Anordnung; Approximativer Attention-Mechanismus (Anchor-Block, Passing
         Blocks, Berechnung). The Portuguese version of the same page,
         "Metodologia: APB-V", says the same.
  [SYS]  same page, "Systemseitige Optimierungen" (fused forward with lse merge,
         load balancing, overlapped communication).
  [LIM]  same page, "Bedeutung und Ansprueche" > Einschraenkungen: on one GPU the
         method reduces to standard FlashAttention.

What the oracle computes, in the pages' order:
  1. the sequence is cut into H contiguous context blocks B^(h)            [METH]
  2. the anchor block B_a is a fixed initial segment                      [METH]
  3. each block forwards a passing block: its most important KV rows,
     ranked by query-to-context attention scores                          [METH]
  4. each block's queries attend over anchor + aggregated passing blocks
     + its own local context                                              [METH]

Readings where the pages are silent (each is listed in the design notes):
  R1 blocks have equal length n_b = N / H (N % H == 0).
  R2 the anchor is tokens [0, A) with A <= n_b; blocks h >= 1 see it; block 0 sees it
     as ordinary local context.
  R3 block 0's passing candidates exclude the anchor rows, so no row is visible twice.
  R4 importance score of key p in block j, KV head g: the mean, over the G query heads
     of group g and the last w queries i of block j, of the causal softmax of
     scale * <q_i, k_p> taken over the block's own keys [s_j, i] only.
  R5 block j passes l_j = min(l, |C_j|) rows: the largest scores, ties to the lower
     position, reported in ascending position order and padded with -1.
  R6 query head hq uses KV head hq // G.
  R7 logits are scale * <q, k> with scale = 1/sqrt(d) unless given.
  R8 a query sees its own key (inclusive causal diagonal).
  R9 the last block's selection is never consumed and is not computed.
  R17 the query block B_qr (text question, after the context) attends exactly to all
     context keys and causally to its own keys; per-host partials over disjoint key
     sets merged by log-sum-exp give exactly that (see query_block_attention).
  R18 (variant) query-aware selection: the observers scoring a block's keys are the
     query block's rows (all G heads), over all of the block's keys; selection rule
     as in R5 (see query_window_scores).

All arithmetic is float64 on the exact values of the stored inputs. Inputs may be
passed as stored (bf16 bit patterns as uint16, or float32/float64); every function
widens exactly the slices it reads. Rows are handled in chunks only to bound memory;
every row's softmax is computed whole, as defined.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# ---------------------------------------------------------------- input widening

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of stored inputs: bf16 bits (uint16) or float32/float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


# ------------------------------------------------------------------ problem shape

@dataclass(frozen=True)
class Shape:
    seq_len: int
    num_hosts: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    anchor_len: int
    passing_len: int
    window: int
    sm_scale: float = 0.0   # <= 0 means 1/sqrt(head_dim)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def block_len(self) -> int:
        return self.seq_len // self.num_hosts

    @property
    def scale(self) -> float:
        return float(self.sm_scale) if self.sm_scale > 0 else 1.0 / np.sqrt(float(self.head_dim))

    def check(self) -> None:
        n, h = self.seq_len, self.num_hosts
        assert h >= 1 and n >= 1 and n % h == 0, "R1: N must split into H equal blocks"
        assert self.num_q_heads % self.num_kv_heads == 0
        assert 0 <= self.anchor_len <= self.block_len, "R2: anchor lies inside block 0"
        assert self.passing_len >= 0
        assert 1 <= self.window <= self.block_len


def shape_of(cfg) -> Shape:
    """Build an oracle Shape from any object with the same field names."""
    return Shape(cfg.seq_len, cfg.num_hosts, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                 cfg.anchor_len, cfg.passing_len, cfg.window)


# ------------------------------------------------------- step 1-2: blocks, anchor

def context_block(sh: Shape, h: int) -> tuple[int, int]:
    """[s_h, e_h) of context block B^(h) (R1) -- [METH] Kontext-Splitting."""
    nb = sh.block_len
    return h * nb, (h + 1) * nb


def anchor_rows(sh: Shape) -> np.ndarray:
    """Positions of the anchor block B_a: the first A tokens (R2) -- [METH] Anchor-Block."""
    return np.arange(sh.anchor_len, dtype=np.int64)


def passing_candidates(sh: Shape, j: int) -> np.ndarray:
    """Rows block j may pass: its own positions, minus the anchor for j == 0 (R3)."""
    s, e = context_block(sh, j)
    lo = max(s, sh.anchor_len) if j == 0 else s
    return np.arange(lo, e, dtype=np.int64)


def passing_length(sh: Shape, j: int) -> int:
    """l_j = min(l, |C_j|) (R5)."""
    return min(sh.passing_len, len(passing_candidates(sh, j)))


# --------------------------------------------------------- step 3: passing blocks

def window_scores(sh: Shape, q: np.ndarray, k: np.ndarray, j: int, g: int) -> np.ndarray:
    """Importance score of every key of block j for KV head g (R4), float64 [n_b].

    [METH] Passing Blocks: the most essential KV rows of a block are found with
    query-to-context attention scores. Observers here are the last w queries of the
    same block, all G query heads of the group; each observer's softmax runs over the
    block's local causal keys only, and the score is the mean probability mass.
    """
    sh.check()
    s, e = context_block(sh, j)
    G, w = sh.group, sh.window
    heads = range(g * G, (g + 1) * G)
    obs_pos = np.arange(e - w, e)                   # observer query positions
    key_pos = np.arange(s, e)                       # local keys of block j
    kl = to_f64(k[s:e, g, :])                       # [n_b, d]
    total = np.zeros(e - s, dtype=np.float64)
    for hq in heads:
        qw = to_f64(q[e - w:e, hq, :])              # [w, d]
        x = sh.scale * (qw @ kl.T)                  # logits [w, n_b]
        visible = key_pos[None, :] <= obs_pos[:, None]
        x = np.where(visible, x, -np.inf)
        m = x.max(axis=1, keepdims=True)
        ex = np.exp(x - m)                          # exp(-inf) = 0 for hidden keys
        z = ex.sum(axis=1, keepdims=True)
        pi = ex / z                                 # each row sums to 1
        total += pi.sum(axis=0)
    return total / (G * w)


def all_window_scores(sh: Shape, q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Scores for every block that passes rows (j < H-1, R9): float64 [H-1, Hkv, n_b]."""
    sh.check()
    H, hkv, nb = sh.num_hosts, sh.num_kv_heads, sh.block_len
    out = np.zeros((max(H - 1, 0), hkv, nb), dtype=np.float64)
    for j in range(H - 1):
        for g in range(hkv):
            out[j, g] = window_scores(sh, q, k, j, g)
    return out


def select_passing(sh: Shape, scores: np.ndarray) -> np.ndarray:
    """Top-l_j rows per (block j, KV head g): int32 [H-1, Hkv, l], ascending, -1 padded.

    Ranking is (score descending, position ascending) (R5). [METH] Passing Blocks.
    """
    H, hkv, l = sh.num_hosts, sh.num_kv_heads, sh.passing_len
    idx = np.full((max(H - 1, 0), hkv, l), -1, dtype=np.int32)
    for j in range(H - 1):
        s, _ = context_block(sh, j)
        cand = passing_candidates(sh, j)
        lj = passing_length(sh, j)
        for g in range(hkv):
            sc = scores[j, g, cand - s]
            order = np.lexsort((cand, -sc))         # primary: -score, then position
            idx[j, g, :lj] = np.sort(cand[order[:lj]])
    return idx


def selection_margins(sh: Shape, scores: np.ndarray) -> np.ndarray:
    """Relative gap between the last selected and the first rejected score, [H-1, Hkv].

    NaN where nothing is rejected (l_j == |C_j|) or nothing is selected.
    """
    H, hkv = sh.num_hosts, sh.num_kv_heads
    out = np.full((max(H - 1, 0), hkv), np.nan)
    for j in range(H - 1):
        s, _ = context_block(sh, j)
        cand = passing_candidates(sh, j)
        lj = passing_length(sh, j)
        if lj == 0 or lj == len(cand):
            continue
        for g in range(hkv):
            sc = np.sort(scores[j, g, cand - s])[::-1]
            out[j, g] = (sc[lj - 1] - sc[lj]) / sc[lj - 1]
    return out


# ------------------------------------------------ step 4: approximate attention

def visible_prefix(sh: Shape, idx: np.ndarray, h: int, g: int) -> np.ndarray:
    """Non-local keys of block h for KV head g: anchor then passing blocks j < h, in order.

    [METH] Berechnung: attention runs over the anchor, the aggregated passing blocks
    and the local context. Block 0 has no non-local keys.
    """
    if h == 0:
        return np.zeros(0, dtype=np.int64)
    parts = [anchor_rows(sh)]
    for j in range(h):
        sel = idx[j, g]
        parts.append(sel[sel >= 0].astype(np.int64))
    return np.concatenate(parts)


def attention_rows(sh: Shape, q, k, v, idx, hq: int, rows: np.ndarray):
    """Output rows O[rows, hq, :] and LSE[hq, rows] (natural log), float64.

    Every listed row must lie in one block. Visible set of query i in block h:
    prefix(h, g) U [s_h, i]; softmax of scale * <q_i, k_p> over it; O = P V.
    """
    rows = np.asarray(rows, dtype=np.int64)
    g = hq // sh.group
    h = int(rows[0] // sh.block_len)
    assert np.all(rows // sh.block_len == h)
    s, e = context_block(sh, h)
    pre = visible_prefix(sh, idx, h, g)
    local = np.arange(s, e, dtype=np.int64)
    keys = np.concatenate([pre, local])
    x = sh.scale * (to_f64(q[rows, hq, :]) @ to_f64(k[keys, g, :]).T)   # [R, L_h + n_b]
    hidden = np.zeros(x.shape, dtype=bool)
    hidden[:, len(pre):] = local[None, :] > rows[:, None]       # causal (R8)
    x = np.where(hidden, -np.inf, x)
    m = x.max(axis=1, keepdims=True)
    ex = np.exp(x - m)
    z = ex.sum(axis=1, keepdims=True)
    o = (ex / z) @ to_f64(v[keys, g, :])
    lse = m[:, 0] + np.log(z[:, 0])
    return o, lse


def approx_attention(sh: Shape, q, k, v, idx, row_chunk: int = 1024):
    """Full output O [N, Hq, d] and LSE [Hq, N], float64."""
    sh.check()
    n, hq_n, d = q.shape
    o = np.zeros((n, hq_n, d), dtype=np.float64)
    lse = np.zeros((hq_n, n), dtype=np.float64)
    for h in range(sh.num_hosts):
        s, e = context_block(sh, h)
        for hq in range(hq_n):
            for r0 in range(s, e, row_chunk):
                rows = np.arange(r0, min(e, r0 + row_chunk))
                o[rows, hq], lse[hq, rows] = attention_rows(sh, q, k, v, idx, hq, rows)
    return o, lse


def visible_count(sh: Shape, idx: np.ndarray, i: int, g: int) -> int:
    """|V(i)| = L_h + (i - s_h + 1) for query position i and KV head g."""
    h = i // sh.block_len
    s, _ = context_block(sh, h)
    return len(visible_prefix(sh, idx, h, g)) + (i - s + 1)


# --------------------------------------------------------------- whole pipeline

def run(sh: Shape, q, k, v, attention: bool = True):
    """Selection then attention on stored inputs; returns a dict of float64 results."""
    scores = all_window_scores(sh, q, k)
    idx = select_passing(sh, scores)
    out = {"scores": scores, "idx": idx, "margins": selection_margins(sh, scores)}
    if attention:
        out["o"], out["lse"] = approx_attention(sh, q, k, v, idx)
    return out


# ------------------------------------------- query block B_qr (fused query forward)

def query_block_attention(sh: Shape, q_qr, k_qr, v_qr, k, v):
    """Attention of the query block B_qr: O [n_qr, Hq, d] and LSE [Hq, n_qr], float64.

    [METH] Kontext-Splitting separates the text query block B_qr from the context
    blocks; [SYS] fused context + query forward: every host attends the query rows to
    what it holds and the partial results are merged with their log-sum-exp. Reading
    (R17): the partial key sets are disjoint (each host's own context block, plus the
    query's own keys), so the merge is exact: query row i sees every context key
    [0, N) and the query keys [0, i] (causal). This function is that plain definition;
    it does not split or merge.
    """
    n_qr = q_qr.shape[0]
    G = sh.group
    o = np.zeros((n_qr, sh.num_q_heads, sh.head_dim))
    lse = np.zeros((sh.num_q_heads, n_qr))
    rows = np.arange(n_qr)
    for hq in range(sh.num_q_heads):
        g = hq // G
        kk = np.concatenate([to_f64(k[:, g, :]), to_f64(k_qr[:, g, :])])
        vv = np.concatenate([to_f64(v[:, g, :]), to_f64(v_qr[:, g, :])])
        x = sh.scale * (to_f64(q_qr[:, hq, :]) @ kk.T)             # [n_qr, N + n_qr]
        hidden = np.zeros(x.shape, dtype=bool)
        hidden[:, sh.seq_len:] = rows[None, :] > rows[:, None]     # causal inside B_qr
        x = np.where(hidden, -np.inf, x)
        m = x.max(axis=1, keepdims=True)
        ex = np.exp(x - m)
        z = ex.sum(axis=1, keepdims=True)
        o[:, hq] = (ex / z) @ vv
        lse[hq] = m[:, 0] + np.log(z[:, 0])
    return o, lse


# ------------------------------------------- query-aware passing selection (variant)

def query_window_scores(sh: Shape, q_qr, k, j: int, g: int) -> np.ndarray:
    """Importance of every key of block j for KV head g, scored by the query block.

    [METH] Passing Blocks: KV rows are ranked by query-to-context attention scores.
    Reading R18 (variant): the observers are the rows of the query block B_qr (all G
    query heads of group g) instead of the block's last w queries. B_qr follows the
    whole context, so every key of block j is visible; each observer's softmax runs
    over block j's keys, and the score is the mean probability mass. float64 [n_b].
    """
    s, e = context_block(sh, j)
    G = sh.group
    n_qr = q_qr.shape[0]
    kl = to_f64(k[s:e, g, :])
    total = np.zeros(e - s, dtype=np.float64)
    for hq in range(g * G, (g + 1) * G):
        x = sh.scale * (to_f64(q_qr[:, hq, :]) @ kl.T)               # [n_qr, n_b]
        m = x.max(axis=1, keepdims=True)
        ex = np.exp(x - m)
        total += (ex / ex.sum(axis=1, keepdims=True)).sum(axis=0)
    return total / (G * n_qr)


def all_query_scores(sh: Shape, q_qr, k) -> np.ndarray:
    """Query-aware scores of every block that passes rows: float64 [H-1, Hkv, n_b]."""
    H, hkv, nb = sh.num_hosts, sh.num_kv_heads, sh.block_len
    out = np.zeros((max(H - 1, 0), hkv, nb), dtype=np.float64)
    for j in range(H - 1):
        for g in range(hkv):
            out[j, g] = query_window_scores(sh, q_qr, k, j, g)
    return out
