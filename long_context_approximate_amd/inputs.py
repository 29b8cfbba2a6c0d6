"""Seeded synthetic inputs for the approximate-attention prefill path.

This module only draws random tensors and stores them in the formats the kernels
read (bf16 bit patterns or float32). It holds none of the method's arithmetic, so
both the fp64 oracle and the HIP path can consume its output without sharing any
computation.

The pages evaluate on long-video benchmarks with trained multimodal models; those
datasets and weights are not available here, so every workload is synthetic:
i.i.d. normal tensors, a low-rank "repeated frames" video stand-in, or heavy-tailed
keys, at the shapes of the named workloads.

Recipe (per tensor stream ``s``: 0 = q, 1 = k, 2 = v, 3 = video basis,
4 = video coefficients): ``numpy.random.default_rng(SeedSequence([seed, s]))``,
float32 standard normals drawn in token order in chunks, rounded to bf16 with
round-to-nearest-even where the workload is bf16. Student-t keys are drawn in
float64, divided by sqrt(3) and rounded to float32 first.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

_CHUNK_TOKENS = 8192


@dataclass(frozen=True)
class SpavaConfig:
    """Shape of one prefill attention layer, batch 1."""

    name: str
    seq_len: int          # N tokens
    num_hosts: int        # H virtual hosts (contiguous context blocks)
    num_q_heads: int      # Hq
    num_kv_heads: int     # Hkv (Hq % Hkv == 0; GQA group size G = Hq / Hkv)
    head_dim: int         # d
    anchor_len: int       # A
    passing_len: int      # l
    window: int           # w, last queries of a block that score its keys
    dtype: str            # "bf16" or "f32"
    dist: str             # "normal", "video" or "student_t3"
    seed: int

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def block_len(self) -> int:
        return self.seq_len // self.num_hosts

    def with_(self, **kw) -> "SpavaConfig":
        return replace(self, **kw)


# The five named workloads. The 64K video workload leaves w unstated; 128 is the
# window of the other >= 64K workloads.
CONFIGS = {
    "tiny_f32_512": SpavaConfig("tiny_f32_512", 512, 2, 2, 2, 64, 32, 16, 16,
                                "f32", "normal", 1001),
    "h4_16k": SpavaConfig("h4_16k", 16384, 4, 28, 4, 128, 1024, 512, 64,
                          "bf16", "normal", 1002),
    "video_h8_64k": SpavaConfig("video_h8_64k", 65536, 8, 28, 4, 128, 2048, 1024, 128,
                                "bf16", "video", 1003),
    "h8_128k": SpavaConfig("h8_128k", 131072, 8, 28, 4, 128, 4096, 2048, 128,
                           "bf16", "normal", 1004),
    "t3_h16_256k": SpavaConfig("t3_h16_256k", 262144, 16, 32, 8, 128, 4096, 2048, 128,
                               "bf16", "student_t3", 1005),
}

# Video stand-in: 10 frames of 6528 tokens share one rank-16 structure per KV head,
# followed by 256 text tokens (65280 + 256 = 65536).
VIDEO_FRAME_TOKENS = 6528
VIDEO_FRAMES = 10
VIDEO_RANK = 16
VIDEO_NOISE = 0.3


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (a format conversion)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _normal_tensor(seed: int, stream: int, shape, dtype: str) -> np.ndarray:
    n_tok = shape[0]
    per_tok = int(np.prod(shape[1:]))
    out = np.empty(shape, np.uint16 if dtype == "bf16" else np.float32)
    flat = out.reshape(n_tok, per_tok)
    rng = _rng(seed, stream)
    for t0 in range(0, n_tok, _CHUNK_TOKENS):
        t1 = min(n_tok, t0 + _CHUNK_TOKENS)
        x = rng.standard_normal((t1 - t0, per_tok), dtype=np.float32)
        flat[t0:t1] = _store(x, dtype)
    return out


def _student_t3_tensor(seed: int, stream: int, shape, dtype: str) -> np.ndarray:
    n_tok = shape[0]
    per_tok = int(np.prod(shape[1:]))
    out = np.empty(shape, np.uint16 if dtype == "bf16" else np.float32)
    flat = out.reshape(n_tok, per_tok)
    rng = _rng(seed, stream)
    for t0 in range(0, n_tok, _CHUNK_TOKENS):
        t1 = min(n_tok, t0 + _CHUNK_TOKENS)
        x = (rng.standard_t(3, (t1 - t0, per_tok)) / np.sqrt(3.0)).astype(np.float32)
        flat[t0:t1] = _store(x, dtype)
    return out


def _video_keys(cfg: SpavaConfig) -> np.ndarray:
    n, hkv, d = cfg.seq_len, cfg.num_kv_heads, cfg.head_dim
    n_video = min(n, VIDEO_FRAMES * VIDEO_FRAME_TOKENS)
    rng_basis = _rng(cfg.seed, 3)
    rng_coef = _rng(cfg.seed, 4)
    rng_noise = _rng(cfg.seed, 1)
    basis = rng_basis.standard_normal((hkv, VIDEO_RANK, d), dtype=np.float32) * np.float32(0.25)
    coef = rng_coef.standard_normal((hkv, VIDEO_FRAME_TOKENS, VIDEO_RANK), dtype=np.float32)
    frame = np.einsum("gtr,grd->tgd", coef, basis).astype(np.float32)  # [6528, Hkv, d]
    out = np.empty((n, hkv, d), np.uint16 if cfg.dtype == "bf16" else np.float32)
    for t0 in range(0, n, _CHUNK_TOKENS):
        t1 = min(n, t0 + _CHUNK_TOKENS)
        noise = rng_noise.standard_normal((t1 - t0, hkv, d), dtype=np.float32)
        tok = np.arange(t0, t1)
        x = noise.copy()
        vid = tok < n_video
        if vid.any():
            x[vid] = frame[tok[vid] % VIDEO_FRAME_TOKENS] + np.float32(VIDEO_NOISE) * noise[vid]
        out[t0:t1] = _store(x, cfg.dtype)
    return out


def make_inputs(cfg: SpavaConfig) -> dict:
    """Return {"q": [N,Hq,d], "k": [N,Hkv,d], "v": [N,Hkv,d]} as stored bits/values.

    bf16 workloads return uint16 bit patterns; f32 workloads return float32.
    """
    n, hq, hkv, d = cfg.seq_len, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    q = _normal_tensor(cfg.seed, 0, (n, hq, d), cfg.dtype)
    if cfg.dist == "normal":
        k = _normal_tensor(cfg.seed, 1, (n, hkv, d), cfg.dtype)
    elif cfg.dist == "student_t3":
        k = _student_t3_tensor(cfg.seed, 1, (n, hkv, d), cfg.dtype)
    elif cfg.dist == "video":
        k = _video_keys(cfg)
    else:
        raise ValueError(f"unknown distribution {cfg.dist!r}")
    v = _normal_tensor(cfg.seed, 2, (n, hkv, d), cfg.dtype)
    return {"q": q, "k": k, "v": v}


def small_config(name="small", seq_len=3000, num_hosts=3, num_q_heads=6, num_kv_heads=2,
                 head_dim=128, anchor_len=100, passing_len=70, window=50, dtype="bf16",
                 dist="normal", seed=7) -> SpavaConfig:
    """A ragged, multi-tile shape for quick parity checks."""
    return SpavaConfig(name, seq_len, num_hosts, num_q_heads, num_kv_heads, head_dim,
                       anchor_len, passing_len, window, dtype, dist, seed)
