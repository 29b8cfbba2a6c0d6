"""The Python binding checks every tensor against the shape before a pointer reaches
the C ABI (a wrong dtype, size or stride would make the kernels read or write outside
the tensor). Each rejection is driven on the CPU: dtype, shape and stride are checked
before device placement, so CPU tensors reach every check, and a tensor that passes
them all is still refused for not being on the GPU."""
from __future__ import annotations

import os

import pytest
import torch

from long_context_approximate_amd import spava

N, H, HQ, HKV, D, A, L, W = 1024, 4, 4, 2, 64, 32, 16, 8


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(spava.LIB_PATH):
        pytest.skip("libspava.so not built")


def _shape(**kw):
    return spava.make_shape(N, H, HQ, HKV, D, A, L, W, **kw)


def _good():
    bf = torch.bfloat16
    return {"q": torch.zeros(N, HQ, D, dtype=bf), "k": torch.zeros(N, HKV, D, dtype=bf),
            "v": torch.zeros(N, HKV, D, dtype=bf), "out": torch.zeros(N, HQ, D, dtype=bf),
            "idx": torch.zeros(H - 1, HKV, L, dtype=torch.int32),
            "scores": torch.zeros(H - 1, HKV, N // H, dtype=torch.float64),
            "lse": torch.zeros(HQ, N, dtype=torch.float32)}


def _attn(t, shape=None):
    return spava.spava_approx_attn_fwd(shape or _shape(), t["q"], t["k"], t["v"], t["idx"],
                                       t["out"], t["lse"])


def _select(t, shape=None):
    return spava.spava_select_passing(shape or _shape(), t["q"], t["k"], t["idx"], t["scores"])


@pytest.mark.parametrize("name,bad,msg", [
    ("q", torch.zeros(N, HQ, D, dtype=torch.float32), "dtype"),
    ("k", torch.zeros(N, HKV + 1, D, dtype=torch.bfloat16), "shape"),
    ("v", torch.zeros(N - 1, HKV, D, dtype=torch.bfloat16), "shape"),
    ("out", torch.zeros(N, HQ, D, dtype=torch.float16), "dtype"),
    ("out", torch.zeros(N, HQ, 2 * D, dtype=torch.bfloat16)[:, :, :D], "stride"),
    ("k", torch.zeros(HKV, N, D, dtype=torch.bfloat16).transpose(0, 1), "stride"),
    ("idx", torch.zeros(H - 1, HKV, L, dtype=torch.int64), "dtype"),
    ("idx", torch.zeros(H - 1, HKV, L - 1, dtype=torch.int32), "shape"),
    ("idx", torch.zeros(H - 1, L, HKV, dtype=torch.int32).transpose(1, 2), "contiguous"),
    ("lse", torch.zeros(N, HQ, dtype=torch.float32), "shape"),
    ("lse", torch.zeros(HQ, N, dtype=torch.float64), "dtype"),
])
def test_attention_rejects_mismatched_tensors(name, bad, msg):
    t = _good()
    t[name] = bad
    with pytest.raises(ValueError, match=msg):
        _attn(t)


@pytest.mark.parametrize("name,bad,msg", [
    ("scores", torch.zeros(H - 1, HKV, N // H, dtype=torch.float32), "dtype"),
    ("scores", torch.zeros(H, HKV, N // H, dtype=torch.float64), "shape"),
    ("idx", torch.zeros(H, HKV, L, dtype=torch.int32), "shape"),
    ("q", torch.zeros(N, HQ, D, dtype=torch.bfloat16)[:, :, None, :].expand(N, HQ, 2, D)
     .reshape(N, HQ * 2, D)[:, :HQ], "stride"),
])
def test_selection_rejects_mismatched_tensors(name, bad, msg):
    t = _good()
    t[name] = bad
    with pytest.raises(ValueError, match=msg):
        _select(t)


def test_float32_shape_wants_float32_tensors():
    t = _good()
    with pytest.raises(ValueError, match="dtype"):
        _attn(t, _shape(dtype=spava.SPAVA_F32))


def test_strided_views_matching_the_shape_pass_to_the_device_check():
    # q and out inside wider [N, Hq, 2d] buffers, described by the shape's strides: every
    # size/stride check passes and only the CPU placement is refused.
    t = _good()
    t["q"] = torch.zeros(N, HQ, 2 * D, dtype=torch.bfloat16)[:, :, :D]
    t["out"] = torch.zeros(N, HQ, 2 * D, dtype=torch.bfloat16)[:, :, :D]
    wide = _shape(strides=(HQ * 2 * D, 2 * D, HKV * D, D, HQ * 2 * D, 2 * D))
    with pytest.raises(ValueError, match="device"):
        _attn(t, wide)


def test_well_formed_cpu_tensors_are_refused_for_their_placement():
    with pytest.raises(ValueError, match="device"):
        _attn(_good())
    with pytest.raises(ValueError, match="device"):
        _select(_good())


def test_query_entries_check_their_tensors():
    t = _good()
    nq = 7
    q_qr = torch.zeros(nq, HQ, D, dtype=torch.bfloat16)
    kv_qr = torch.zeros(nq, HKV, D, dtype=torch.bfloat16)
    out_qr = torch.zeros(nq, HQ, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="lse_qr: shape"):
        spava.spava_query_attn_fwd(_shape(), q_qr, kv_qr, kv_qr, t["k"], t["v"], out_qr,
                                   torch.zeros(HQ, N, dtype=torch.float32))
    with pytest.raises(ValueError, match="out: shape"):
        spava.spava_query_attn_fwd(_shape(), q_qr, kv_qr, kv_qr, t["k"], t["v"], t["out"])
    with pytest.raises(ValueError, match="k: shape"):
        spava.spava_select_passing_query(_shape(), q_qr, kv_qr, t["idx"])
    with pytest.raises(ValueError, match="device"):
        spava.spava_select_passing_query(_shape(), q_qr, t["k"], t["idx"])


def test_caller_workspace_must_be_large_enough():
    t = _good()
    need = spava.spava_attn_workspace_bytes(_shape())
    with pytest.raises(ValueError, match="workspace"):
        spava.spava_approx_attn_fwd(_shape(), t["q"], t["k"], t["v"], t["idx"], t["out"], None,
                                    torch.zeros(need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace: dtype"):
        spava.spava_approx_attn_fwd(_shape(), t["q"], t["k"], t["v"], t["idx"], t["out"], None,
                                    torch.zeros(need, dtype=torch.int8))
