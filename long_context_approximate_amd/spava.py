"""ctypes binding over the C ABI in include/spava.h (argument marshalling only).

Every step of the path runs in libspava.so's HIP kernels; this module only turns
torch tensors into device pointers, sizes the caller-owned workspace and raises on
a non-OK status. There is no CPU fallback: if the library is missing, loading it
raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_NAME = "libspava.so"
LIB_PATH = os.environ.get("SPAVA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                       LIB_NAME)

SPAVA_BF16 = 0
SPAVA_F32 = 1

# Every symbol include/spava.h declares.
EXPORTS = (
    "spava_status_string",
    "spava_abi_version",
    "spava_validate_shape",
    "spava_select_workspace_bytes",
    "spava_attn_workspace_bytes",
    "spava_select_passing",
    "spava_approx_attn_fwd",
    "spava_query_workspace_bytes",
    "spava_query_attn_fwd",
    "spava_select_query_workspace_bytes",
    "spava_select_passing_query",
    "spava_layer_overlap_workspace_bytes",
    "spava_layer_overlap_fwd",
)


class SpavaShape(ctypes.Structure):
    """Mirror of spava_shape."""

    _fields_ = [
        ("seq_len", ctypes.c_int64),
        ("num_hosts", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("anchor_len", ctypes.c_int32),
        ("passing_len", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_double),
        ("q_stride_tok", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("kv_stride_tok", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64),
        ("o_stride_tok", ctypes.c_int64),
        ("o_stride_head", ctypes.c_int64),
    ]


class SpavaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libspava.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(p)
    vp, sz, i32p, f64p, f32p = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p)
    shp = ctypes.POINTER(SpavaShape)
    lib.spava_status_string.argtypes = [ctypes.c_int]
    lib.spava_status_string.restype = ctypes.c_char_p
    lib.spava_abi_version.argtypes = []
    lib.spava_abi_version.restype = ctypes.c_int
    lib.spava_validate_shape.argtypes = [shp]
    lib.spava_validate_shape.restype = ctypes.c_int
    lib.spava_select_workspace_bytes.argtypes = [shp, ctypes.POINTER(ctypes.c_size_t)]
    lib.spava_select_workspace_bytes.restype = ctypes.c_int
    lib.spava_attn_workspace_bytes.argtypes = [shp, ctypes.POINTER(ctypes.c_size_t)]
    lib.spava_attn_workspace_bytes.restype = ctypes.c_int
    lib.spava_select_passing.argtypes = [shp, vp, vp, i32p, f64p, vp, sz, vp]
    lib.spava_select_passing.restype = ctypes.c_int
    lib.spava_approx_attn_fwd.argtypes = [shp, vp, vp, vp, i32p, vp, f32p, vp, sz, vp]
    lib.spava_approx_attn_fwd.restype = ctypes.c_int
    lib.spava_query_workspace_bytes.argtypes = [shp, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]
    lib.spava_query_workspace_bytes.restype = ctypes.c_int
    lib.spava_query_attn_fwd.argtypes = [shp, ctypes.c_int64, vp, vp, vp, vp, vp, vp, f32p, vp, sz,
                                         vp]
    lib.spava_query_attn_fwd.restype = ctypes.c_int
    lib.spava_select_query_workspace_bytes.argtypes = [shp, ctypes.c_int64,
                                                       ctypes.POINTER(ctypes.c_size_t)]
    lib.spava_select_query_workspace_bytes.restype = ctypes.c_int
    lib.spava_select_passing_query.argtypes = [shp, ctypes.c_int64, vp, vp, i32p, f64p, vp, sz, vp]
    lib.spava_select_passing_query.restype = ctypes.c_int
    lib.spava_layer_overlap_workspace_bytes.argtypes = [shp, ctypes.POINTER(ctypes.c_size_t)]
    lib.spava_layer_overlap_workspace_bytes.restype = ctypes.c_int
    lib.spava_layer_overlap_fwd.argtypes = [shp, vp, vp, vp, i32p, f64p, vp, f32p, vp, sz, vp, vp]
    lib.spava_layer_overlap_fwd.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().spava_status_string(status).decode()


def _check(status: int) -> None:
    if status != 0:
        raise SpavaError(status, status_string(status))


def make_shape(seq_len, num_hosts, num_q_heads, num_kv_heads, head_dim, anchor_len,
               passing_len, window, dtype=SPAVA_BF16, sm_scale=0.0, strides=None) -> SpavaShape:
    """Shape with dense [N, heads, d] strides unless `strides` (6 ints) is given."""
    if strides is None:
        strides = (num_q_heads * head_dim, head_dim, num_kv_heads * head_dim, head_dim,
                   num_q_heads * head_dim, head_dim)
    return SpavaShape(seq_len, num_hosts, num_q_heads, num_kv_heads, head_dim, anchor_len,
                      passing_len, window, dtype, sm_scale, *strides)


def shape_from_config(cfg, sm_scale=0.0) -> SpavaShape:
    dt = SPAVA_BF16 if cfg.dtype == "bf16" else SPAVA_F32
    return make_shape(cfg.seq_len, cfg.num_hosts, cfg.num_q_heads, cfg.num_kv_heads,
                      cfg.head_dim, cfg.anchor_len, cfg.passing_len, cfg.window, dt, sm_scale)


def validate_shape(shape: SpavaShape) -> int:
    return load().spava_validate_shape(ctypes.byref(shape))


def spava_select_workspace_bytes(shape: SpavaShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load().spava_select_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def spava_attn_workspace_bytes(shape: SpavaShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load().spava_attn_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _workspace(nbytes: int, device, workspace=None):
    import torch
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def spava_select_passing(shape: SpavaShape, q, k, passing_idx, scores_out=None,
                         workspace=None, stream=None):
    """Write passing_idx (int32 [H-1, Hkv, l]) and optionally scores_out (f64 [H-1, Hkv, n_b])."""
    nbytes = spava_select_workspace_bytes(shape)
    ws = _workspace(nbytes, q.device, workspace)
    _check(load().spava_select_passing(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(passing_idx),
                                       _ptr(scores_out), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)))
    return ws


def spava_approx_attn_fwd(shape: SpavaShape, q, k, v, passing_idx, out, lse_out=None,
                          workspace=None, stream=None):
    """Write out ([N, Hq, d]) and optionally lse_out (f32 [Hq, N])."""
    nbytes = spava_attn_workspace_bytes(shape)
    ws = _workspace(nbytes, q.device, workspace)
    _check(load().spava_approx_attn_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(passing_idx), _ptr(out), _ptr(lse_out), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)))
    return ws


def spava_select_query_workspace_bytes(shape: SpavaShape, n_query: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().spava_select_query_workspace_bytes(ctypes.byref(shape), n_query,
                                                     ctypes.byref(n)))
    return n.value


def spava_select_passing_query(shape: SpavaShape, q_qr, k, passing_idx, scores_out=None,
                               workspace=None, stream=None):
    """Query-aware selection: observers are the rows of q_qr ([n_query, Hq, d])."""
    n_query = q_qr.shape[0]
    nbytes = spava_select_query_workspace_bytes(shape, n_query)
    ws = _workspace(nbytes, q_qr.device, workspace)
    _check(load().spava_select_passing_query(ctypes.byref(shape), n_query, _ptr(q_qr), _ptr(k),
                                             _ptr(passing_idx), _ptr(scores_out), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(stream)))
    return ws


def spava_query_workspace_bytes(shape: SpavaShape, n_query: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().spava_query_workspace_bytes(ctypes.byref(shape), n_query, ctypes.byref(n)))
    return n.value


def spava_query_attn_fwd(shape: SpavaShape, q_qr, k_qr, v_qr, k, v, out_qr, lse_qr=None,
                         workspace=None, stream=None):
    """Write out_qr ([n_query, Hq, d]) and optionally lse_qr (f32 [Hq, n_query])."""
    n_query = q_qr.shape[0]
    nbytes = spava_query_workspace_bytes(shape, n_query)
    ws = _workspace(nbytes, q_qr.device, workspace)
    _check(load().spava_query_attn_fwd(ctypes.byref(shape), n_query, _ptr(q_qr), _ptr(k_qr),
                                       _ptr(v_qr), _ptr(k), _ptr(v), _ptr(out_qr), _ptr(lse_qr),
                                       _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return ws


def spava_layer_overlap_workspace_bytes(shape: SpavaShape) -> int:
    n = ctypes.c_size_t(0)
    _check(load().spava_layer_overlap_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def spava_layer_overlap_fwd(shape: SpavaShape, q, k, v, passing_idx, out, lse_out=None,
                            scores_out=None, workspace=None, stream=None, side_stream=None):
    """Selection + attention of one layer, the selection on side_stream overlapped with
    the passing-independent attention on stream."""
    nbytes = spava_layer_overlap_workspace_bytes(shape)
    ws = _workspace(nbytes, q.device, workspace)
    main = _stream(stream)
    side = side_stream.cuda_stream if side_stream is not None else None
    if side is None:
        raise ValueError("side_stream is required (a torch.cuda.Stream)")
    _check(load().spava_layer_overlap_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(passing_idx), _ptr(scores_out), _ptr(out),
                                          _ptr(lse_out), _ptr(ws), ws.numel() * ws.element_size(),
                                          main, side))
    return ws


def device_tensors(x: dict, device="cuda"):
    """Move stored inputs (uint16 bf16 bits or float32 numpy arrays) to the GPU."""
    import numpy as np
    import torch
    out = {}
    for name, arr in x.items():
        if arr.dtype == np.uint16:
            out[name] = torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            out[name] = torch.from_numpy(arr).to(device)
    return out


def run_layer(shape: SpavaShape, q, k, v, want_scores=False, want_lse=True, stream=None):
    """Selection then attention on device tensors; returns a dict of device tensors."""
    import torch
    H, hkv, l = shape.num_hosts, shape.num_kv_heads, shape.passing_len
    nb = shape.seq_len // H
    dev = q.device
    idx = torch.empty((max(H - 1, 0), hkv, l), dtype=torch.int32, device=dev)
    scores = (torch.empty((max(H - 1, 0), hkv, nb), dtype=torch.float64, device=dev)
              if want_scores else None)
    spava_select_passing(shape, q, k, idx, scores, stream=stream)
    out = torch.empty((shape.seq_len, shape.num_q_heads, shape.head_dim), dtype=q.dtype,
                      device=dev)
    lse = (torch.empty((shape.num_q_heads, shape.seq_len), dtype=torch.float32, device=dev)
           if want_lse else None)
    spava_approx_attn_fwd(shape, q, k, v, idx, out, lse, stream=stream)
    return {"idx": idx, "scores": scores, "out": out, "lse": lse}
