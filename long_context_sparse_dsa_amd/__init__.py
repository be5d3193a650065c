"""long_context_sparse_dsa_amd -- Python binding of libdsa.so, the gfx950 Gated DSA library.

The functions below carry the names of the C entry points in include/dsa.h
and only marshal arguments: they check dtypes, devices and contiguity,
allocate outputs and workspaces with torch (device memory is the only thing
torch provides), and pass raw pointers plus torch's current HIP stream.
Every step of the layer runs in the library's HIP kernels.  There is no
fallback: if libdsa.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

DSA_KEY_BF16 = 0
DSA_KEY_FP8_E4M3 = 1
_STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
           3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}

EXPORTS = [
    "dsa_version", "dsa_last_error",
    "dsa_index_scores",
    "dsa_topk_workspace_size", "dsa_topk",
    "dsa_sparse_attn_workspace_size", "dsa_sparse_attn",
    "dsa_layer_decode_workspace_size", "dsa_layer_decode", "dsa_set_indexer_events",
    "dsa_set_topk_counters",
    "dsa_layer_prefill_workspace_size", "dsa_layer_prefill",
]

_lib = None


class DSAError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} -> {_STATUS.get(status, status)}: {msg}")
        self.status = status


def load(path: str | None = None):
    """Load libdsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it first "
                           "(python -m long_context_sparse_dsa_amd.build)")
    lib = ctypes.CDLL(path)
    P, I, L, F, S = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                     ctypes.c_size_t)
    lib.dsa_version.restype = ctypes.c_char_p
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_index_scores.argtypes = [P, P, L, P, I, P, I, I, P, P, P, I, I, I, I, P, L, P]
    lib.dsa_topk_workspace_size.argtypes = [I, I, I, I]
    lib.dsa_topk_workspace_size.restype = S
    lib.dsa_topk.argtypes = [P, L, P, P, I, I, I, I, I, P, P, S, P]
    lib.dsa_sparse_attn_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.dsa_sparse_attn_workspace_size.restype = S
    lib.dsa_sparse_attn.argtypes = [P, P, P, P, I, I, P, F, I, I, P, P, P, I, I, I, I, P, P, P,
                                    S, P]
    lib.dsa_layer_decode_workspace_size.argtypes = [I, I, I, I, I]
    lib.dsa_layer_decode_workspace_size.restype = S
    lib.dsa_layer_decode.argtypes = [P, P, L, P, I, P, I, I, P, P, P, P, F, I, I, I, P, P, I, I,
                                     P, P, P, S, P]
    lib.dsa_layer_prefill_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.dsa_layer_prefill_workspace_size.restype = S
    lib.dsa_layer_prefill.argtypes = [P, P, L, P, I, P, I, I, P, P, P, P, F, I, I, I, P, P, P,
                                      I, I, I, I, P, P, P, S, P]
    lib.dsa_set_indexer_events.argtypes = [P, P]
    lib.dsa_set_topk_counters.argtypes = [P]
    for fn in ("dsa_index_scores", "dsa_topk", "dsa_sparse_attn", "dsa_layer_decode",
               "dsa_layer_prefill", "dsa_set_indexer_events", "dsa_set_topk_counters"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name, dtypes, ndim=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _call(fn, *args):
    lib = load()
    st = getattr(lib, fn)(*args)
    if st != 0:
        raise DSAError(fn, st, lib.dsa_last_error().decode())


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _host_max(x, given):
    return int(given) if given is not None else int(x.max().item())


BF16 = (torch.bfloat16,)
KEYS = (torch.bfloat16, torch.float8_e4m3fn)


def _key_dtype(k_idx):
    return DSA_KEY_FP8_E4M3 if k_idx.dtype == torch.float8_e4m3fn else DSA_KEY_BF16


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def dsa_version() -> str:
    return load().dsa_version().decode()


def dsa_last_error() -> str:
    return load().dsa_last_error().decode()


def dsa_index_scores(q_idx, w, k_idx, k_scale, ctx_len, cu_ctx, cu_q=None, max_q=None,
                     max_ctx=None, scores=None, w_ld=None, stream=None):
    """Indexer scores [T, ld] fp32 (entries past each query's position untouched)."""
    _check(q_idx, "q_idx", BF16, 3)
    _check(w, "w", BF16)
    _check(k_idx, "k_idx", KEYS, 2)
    _check(k_scale, "k_scale", (torch.float32,), 1)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    _check(cu_q, "cu_q", (torch.int32,), 1)
    T, H_I, d_I = q_idx.shape
    B = ctx_len.shape[0]
    max_ctx = _host_max(ctx_len, max_ctx)
    if cu_q is not None and max_q is None:
        max_q = int((cu_q[1:] - cu_q[:-1]).max().item())
    if scores is None:
        scores = torch.empty(T, max_ctx, dtype=torch.float32, device=q_idx.device)
    _check(scores, "scores", (torch.float32,), 2)
    if w_ld is None:
        w_ld = 0 if w.dim() == 1 else w.shape[-1]
    _call("dsa_index_scores", _p(q_idx), _p(w), w_ld, _p(k_idx), _key_dtype(k_idx), _p(k_scale),
          H_I, d_I, _p(cu_q), _p(ctx_len), _p(cu_ctx), B, T, max_q or 1, max_ctx, _p(scores),
          scores.stride(0), _stream(stream))
    return scores


def dsa_topk(scores, K, ctx_len, cu_q=None, max_q=None, max_ctx=None, idx=None, stream=None):
    """Exact Top-K positions per row, ascending, -1 padded: int32 [T, K]."""
    _check(scores, "scores", (torch.float32,), 2)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_q, "cu_q", (torch.int32,), 1)
    T = scores.shape[0]
    B = ctx_len.shape[0]
    max_ctx = _host_max(ctx_len, max_ctx)
    if cu_q is not None and max_q is None:
        max_q = int((cu_q[1:] - cu_q[:-1]).max().item())
    if idx is None:
        idx = torch.empty(T, K, dtype=torch.int32, device=scores.device)
    _check(idx, "idx", (torch.int32,), 2)
    nbytes = load().dsa_topk_workspace_size(B, T, max_ctx, K)
    ws = _workspace(nbytes, scores.device)
    _call("dsa_topk", _p(scores), scores.stride(0), _p(cu_q), _p(ctx_len), B, T, max_q or 1,
          max_ctx, K, _p(idx), _p(ws), ws.numel(), _stream(stream))
    return idx


def dsa_sparse_attn(q, k_cache, v_cache, idx, ctx_len, cu_ctx, window=0, gate=None, sm_scale=0.0,
                    cu_q=None, max_q=None, max_ctx=None, out=None, lse=None, stream=None):
    """Gated sparse attention; returns out bf16 [T, Hq, D] (and fills lse if given)."""
    _check(q, "q", BF16, 3)
    _check(k_cache, "k_cache", BF16, 2)
    _check(v_cache, "v_cache", BF16, 2)
    _check(idx, "idx", (torch.int32,), 2)
    _check(gate, "gate", BF16, 3)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    _check(cu_q, "cu_q", (torch.int32,), 1)
    _check(lse, "lse", (torch.float32,), 2)
    T, Hq, D = q.shape
    B = ctx_len.shape[0]
    K = 0 if idx is None else idx.shape[1]
    max_ctx = _host_max(ctx_len, max_ctx)
    if cu_q is not None and max_q is None:
        max_q = int((cu_q[1:] - cu_q[:-1]).max().item())
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", BF16, 3)
    nbytes = load().dsa_sparse_attn_workspace_size(B, T, K, window, Hq, D)
    ws = _workspace(nbytes, q.device)
    _call("dsa_sparse_attn", _p(q), _p(k_cache), _p(v_cache), _p(idx), K, window, _p(gate),
          float(sm_scale), Hq, D, _p(cu_q), _p(ctx_len), _p(cu_ctx), B, T, max_q or 1, max_ctx,
          _p(out), _p(lse), _p(ws), ws.numel(), _stream(stream))
    return out


def prepare_sparse_attn(q, k_cache, v_cache, idx, ctx_len, cu_ctx, max_ctx, out, window=0,
                        gate=None, sm_scale=0.0, ws=None, stream=None):
    """Marshal one dsa_sparse_attn call (one new query per sequence) once;
    returns a no-argument callable that re-issues it (one ctypes call).  The
    tensors must stay alive and unchanged in shape while the callable is used."""
    _check(q, "q", BF16, 3)
    _check(k_cache, "k_cache", BF16, 2)
    _check(v_cache, "v_cache", BF16, 2)
    _check(idx, "idx", (torch.int32,), 2)
    _check(gate, "gate", BF16, 3)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    _check(out, "out", BF16, 3)
    T, Hq, D = q.shape
    B = ctx_len.shape[0]
    K = 0 if idx is None else idx.shape[1]
    nbytes = load().dsa_sparse_attn_workspace_size(B, T, K, window, Hq, D)
    if ws is None:
        ws = _workspace(nbytes, q.device)
    fn = load().dsa_sparse_attn
    args = (_p(q), _p(k_cache), _p(v_cache), _p(idx), K, window, _p(gate), float(sm_scale), Hq,
            D, None, _p(ctx_len), _p(cu_ctx), B, T, 1, int(max_ctx), _p(out), None, _p(ws),
            ws.numel(), _stream(stream))

    def call():
        st = fn(*args)
        if st != 0:
            raise DSAError("dsa_sparse_attn", st, dsa_last_error())
    call.workspace = ws
    return call


def dsa_layer_decode_workspace_size(B, max_ctx, K, Hq, D) -> int:
    return int(load().dsa_layer_decode_workspace_size(B, max_ctx, K, Hq, D))


def dsa_layer_decode(q_idx, w, k_idx, k_scale, q, k_cache, v_cache, gate, K, ctx_len, cu_ctx,
                     max_ctx=None, sm_scale=0.0, out=None, idx_out=None, ws=None, w_ld=None,
                     stream=None):
    """Whole layer for one new query per sequence; returns out bf16 [B, Hq, D]."""
    _check(q_idx, "q_idx", BF16, 3)
    _check(w, "w", BF16)
    _check(k_idx, "k_idx", KEYS, 2)
    _check(k_scale, "k_scale", (torch.float32,), 1)
    _check(q, "q", BF16, 3)
    _check(k_cache, "k_cache", BF16, 2)
    _check(v_cache, "v_cache", BF16, 2)
    _check(gate, "gate", BF16, 3)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    _check(idx_out, "idx_out", (torch.int32,), 2)
    B, H_I, d_I = q_idx.shape
    _, Hq, D = q.shape
    max_ctx = _host_max(ctx_len, max_ctx)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", BF16, 3)
    if ws is None:
        ws = _workspace(dsa_layer_decode_workspace_size(B, max_ctx, K, Hq, D), q.device)
    if w_ld is None:
        w_ld = 0 if w.dim() == 1 else w.shape[-1]
    _call("dsa_layer_decode", _p(q_idx), _p(w), w_ld, _p(k_idx), _key_dtype(k_idx), _p(k_scale),
          H_I, d_I, _p(q), _p(k_cache), _p(v_cache), _p(gate), float(sm_scale), Hq, D, K,
          _p(ctx_len), _p(cu_ctx), B, max_ctx, _p(out), _p(idx_out), _p(ws), ws.numel(),
          _stream(stream))
    return out


def prepare_layer_decode(q_idx, w, k_idx, k_scale, q, k_cache, v_cache, gate, K, ctx_len, cu_ctx,
                         max_ctx, out, ws, sm_scale=0.0, idx_out=None, w_ld=None, stream=None):
    """Marshal one dsa_layer_decode call once; returns a no-argument callable
    that re-issues it (one ctypes call, no per-call argument checks).  The
    tensors must stay alive and unchanged in shape while the callable is used."""
    _check(q_idx, "q_idx", BF16, 3)
    _check(w, "w", BF16)
    _check(k_idx, "k_idx", KEYS, 2)
    _check(k_scale, "k_scale", (torch.float32,), 1)
    _check(q, "q", BF16, 3)
    _check(k_cache, "k_cache", BF16, 2)
    _check(v_cache, "v_cache", BF16, 2)
    _check(gate, "gate", BF16, 3)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    _check(out, "out", BF16, 3)
    _check(idx_out, "idx_out", (torch.int32,), 2)
    B, H_I, d_I = q_idx.shape
    _, Hq, D = q.shape
    if w_ld is None:
        w_ld = 0 if w.dim() == 1 else w.shape[-1]
    fn = load().dsa_layer_decode
    args = (_p(q_idx), _p(w), w_ld, _p(k_idx), _key_dtype(k_idx), _p(k_scale), H_I, d_I, _p(q),
            _p(k_cache), _p(v_cache), _p(gate), float(sm_scale), Hq, D, K, _p(ctx_len),
            _p(cu_ctx), B, int(max_ctx), _p(out), _p(idx_out), _p(ws), ws.numel(),
            _stream(stream))

    def call():
        st = fn(*args)
        if st != 0:
            raise DSAError("dsa_layer_decode", st, dsa_last_error())
    return call


def dsa_set_indexer_events(start, stop):
    """Record the caller's HIP events (raw hipEvent_t handles as ints, or
    None, None) around the indexer launch of later dsa_layer_decode calls
    on this thread."""
    _call("dsa_set_indexer_events", start, stop)


def dsa_set_topk_counters(counters):
    """Count, per Top-K row on this thread, the path that produced it into a
    caller-owned uint32 [5] device tensor (certified union, exact fallback,
    direct, row sweeps, and of those the sampled-threshold ones); None stops
    counting."""
    if counters is not None:
        assert counters.dtype == torch.int32
        assert counters.is_cuda and counters.numel() >= 5 and counters.is_contiguous()
    _call("dsa_set_topk_counters", None if counters is None else counters.data_ptr())


def dsa_layer_prefill_workspace_size(B, T, max_ctx, K, Hq, D) -> int:
    return int(load().dsa_layer_prefill_workspace_size(B, T, max_ctx, K, Hq, D))


def dsa_layer_prefill(q_idx, w, k_idx, k_scale, q, k_cache, v_cache, gate, K, cu_q, ctx_len,
                      cu_ctx, max_q=None, max_ctx=None, sm_scale=0.0, out=None, idx_out=None,
                      ws=None, w_ld=None, stream=None):
    """Whole layer for a chunk of new queries per sequence; returns out bf16 [T, Hq, D]."""
    _check(q_idx, "q_idx", BF16, 3)
    _check(w, "w", BF16)
    _check(k_idx, "k_idx", KEYS, 2)
    _check(k_scale, "k_scale", (torch.float32,), 1)
    _check(q, "q", BF16, 3)
    _check(k_cache, "k_cache", BF16, 2)
    _check(v_cache, "v_cache", BF16, 2)
    _check(gate, "gate", BF16, 3)
    _check(cu_q, "cu_q", (torch.int32,), 1)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    _check(idx_out, "idx_out", (torch.int32,), 2)
    T, H_I, d_I = q_idx.shape
    _, Hq, D = q.shape
    B = ctx_len.shape[0]
    max_ctx = _host_max(ctx_len, max_ctx)
    if max_q is None:
        max_q = int((cu_q[1:] - cu_q[:-1]).max().item())
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", BF16, 3)
    if ws is None:
        ws = _workspace(dsa_layer_prefill_workspace_size(B, T, max_ctx, K, Hq, D), q.device)
    if w_ld is None:
        w_ld = 0 if w.dim() == 1 else w.shape[-1]
    _call("dsa_layer_prefill", _p(q_idx), _p(w), w_ld, _p(k_idx), _key_dtype(k_idx),
          _p(k_scale), H_I, d_I, _p(q), _p(k_cache), _p(v_cache), _p(gate), float(sm_scale), Hq,
          D, K, _p(cu_q), _p(ctx_len), _p(cu_ctx), B, T, max_q, max_ctx, _p(out), _p(idx_out),
          _p(ws), ws.numel(), _stream(stream))
    return out
