"""long_context_sparse_dsa_amd -- Python binding of libdsa.so, the gfx950 Gated DSA library.

The functions below carry the names of the C entry points in include/dsa.h
and only marshal arguments: they check dtypes, devices and contiguity,
allocate outputs and workspaces with torch (device memory is the only thing
torch provides), and pass raw pointers plus torch's current HIP stream.
Every step of the layer runs in the library's HIP kernels.  There is no
fallback: if libdsa.so is missing or fails to load, every call raises.

Shapes are checked on the host before the call (the C ABI sees only
pointers).  `max_ctx` / `max_q` are host bounds used for grid sizing; when
they are omitted the wrappers read them from the device descriptor, a
Python-side convenience that synchronises with the device (the C entry
points themselves never synchronise).  Workspaces allocated here on behalf
of a call on a non-current stream are kept alive for that stream's work.
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
    "dsa_index_scores", "dsa_cache_append",
    "dsa_topk_workspace_size", "dsa_topk",
    "dsa_sparse_attn_workspace_size", "dsa_sparse_attn", "dsa_swa_decode_layers",
    "dsa_layer_decode_workspace_size", "dsa_layer_decode", "dsa_set_indexer_events",
    "dsa_layer_decode_noalloc_max_bytes", "dsa_layer_decode_noalloc", "dsa_layer_decode_append",
    "dsa_set_topk_counters", "dsa_check_index_rows", "dsa_set_index_checks",
    "dsa_layer_prefill_workspace_size", "dsa_layer_prefill_min_workspace_size",
    "dsa_layer_prefill",
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
    path = path or os.environ.get("DSA_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it first "
                           "(python -m long_context_sparse_dsa_amd.build)")
    lib = ctypes.CDLL(path)
    P, I, L, F, S = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                     ctypes.c_size_t)
    lib.dsa_version.restype = ctypes.c_char_p
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_index_scores.argtypes = [P, I, P, P, L, P, I, P, I, I, P, P, P, I, I, I, I, P, L, P]
    lib.dsa_cache_append.argtypes = [P, I, P, P, I, P, P, P, I, I, P, I, P, P, P, P]
    lib.dsa_topk_workspace_size.argtypes = [I, I, I, I]
    lib.dsa_topk_workspace_size.restype = S
    lib.dsa_topk.argtypes = [P, L, P, P, I, I, I, I, I, P, P, S, P]
    lib.dsa_sparse_attn_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.dsa_sparse_attn_workspace_size.restype = S
    lib.dsa_sparse_attn.argtypes = [P, P, P, P, I, I, P, L, F, I, I, P, P, P, I, I, I, I, P, P,
                                    P, S, P]
    lib.dsa_swa_decode_layers.argtypes = [I, P, P, P, P, L, I, F, I, I, P, P, I, I, P, P]
    lib.dsa_layer_decode_workspace_size.argtypes = [I, I, I, I, I]
    lib.dsa_layer_decode_workspace_size.restype = S
    lib.dsa_layer_decode.argtypes = [P, P, L, P, I, P, I, I, P, P, P, P, L, F, I, I, I, P, P, I,
                                     I, P, P, P, S, P]
    lib.dsa_layer_prefill_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.dsa_layer_prefill_workspace_size.restype = S
    lib.dsa_layer_prefill_min_workspace_size.argtypes = [I, I, I, I, I]
    lib.dsa_layer_prefill_min_workspace_size.restype = S
    lib.dsa_layer_prefill.argtypes = [P, I, P, P, L, P, I, P, I, I, P, P, P, P, L, F, I, I, I, P,
                                      P, P, I, I, I, I, P, P, P, S, P]
    lib.dsa_layer_decode_append.argtypes = [P, P, L, P, I, P, I, I, P, P, P, P, L, F, I, I, I,
                                            P, P, I, I, P, P, P, P, P, P, S, P]
    lib.dsa_layer_decode_noalloc_max_bytes.argtypes = []
    lib.dsa_layer_decode_noalloc_max_bytes.restype = S
    lib.dsa_layer_decode_noalloc.argtypes = [P, P, L, P, I, P, I, I, P, P, P, P, L, F, I, I, I,
                                             P, P, I, I, P, P, P]
    lib.dsa_set_indexer_events.argtypes = [P, P]
    lib.dsa_set_topk_counters.argtypes = [P]
    lib.dsa_check_index_rows.argtypes = [P, I, P, P, I, I, I, P, P]
    lib.dsa_set_index_checks.argtypes = [P]
    for fn in ("dsa_index_scores", "dsa_cache_append", "dsa_topk", "dsa_sparse_attn",
               "dsa_swa_decode_layers",
               "dsa_layer_decode",
               "dsa_layer_decode_noalloc", "dsa_layer_decode_append",
               "dsa_layer_prefill", "dsa_set_indexer_events", "dsa_set_topk_counters",
               "dsa_check_index_rows", "dsa_set_index_checks"):
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


def _keep_for(stream, *tensors):
    """Tensors allocated here for work enqueued on `stream`: when that is not
    the current stream, tell the caching allocator so that their memory is not
    handed to later work before the stream's work is done."""
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _shape(t, name, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _gate_stride(gate, T, Hq, D):
    """1 for an elementwise gate [T, Hq, D], 0 for one gate per head [T, Hq]."""
    if gate is None:
        return 1
    if gate.dim() == 3:
        _shape(gate, "gate", (T, Hq, D))
        return 1
    _shape(gate, "gate", (T, Hq))
    return 0


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
    """Host bound of a device descriptor; reading it synchronises (convenience)."""
    return int(given) if given is not None else int(x.max().item())


def _host_max_q(cu_q, given):
    """Largest per-sequence query count; reading it synchronises (convenience)."""
    return int(given) if given is not None else int((cu_q[1:] - cu_q[:-1]).max().item())


def _check_desc(ctx_len, cu_ctx, cu_q, T):
    B = ctx_len.shape[0]
    _shape(cu_ctx, "cu_ctx", (B + 1,))
    _shape(cu_q, "cu_q", (B + 1,))
    if cu_q is None and T != B:
        raise ValueError(f"one query per sequence (no cu_q): {T} rows for {B} sequences")
    return B


def _check_w(w, T, H_I):
    if w.dim() == 1:
        _shape(w, "w", (H_I,))
    else:
        _shape(w, "w", (T, H_I))


def _check_keys(k_idx, k_scale, d_I):
    if k_idx.shape[1] != d_I:
        raise ValueError(f"k_idx: rows of {k_idx.shape[1]}, expected {d_I}")
    if k_idx.dtype == torch.float8_e4m3fn:
        if k_scale is None:
            raise ValueError("fp8 indexer keys need k_scale")
        _shape(k_scale, "k_scale", (k_idx.shape[0],))
    elif k_scale is not None:
        raise ValueError("bf16 indexer keys take no k_scale")


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


def _check_q(q_idx, q_scale):
    """Query-head dtype code; fp8 (E4M3FN) heads carry q_scale fp32 [T, H_I]."""
    _check(q_idx, "q_idx", KEYS, 3)
    _check(q_scale, "q_scale", (torch.float32,), 2)
    if q_idx.dtype == torch.float8_e4m3fn:
        if q_scale is None:
            raise ValueError("fp8 query heads need q_scale [T, H_I]")
        _shape(q_scale, "q_scale", q_idx.shape[:2])
        return 1
    if q_scale is not None:
        raise ValueError("bf16 query heads take no q_scale")
    return 0


def dsa_index_scores(q_idx, w, k_idx, k_scale, ctx_len, cu_ctx, cu_q=None, max_q=None,
                     max_ctx=None, scores=None, w_ld=None, stream=None, q_scale=None):
    """Indexer scores [T, ld] fp32 (entries past each query's position untouched).
    q_idx is bf16, or E4M3FN with q_scale [T, H_I] (prefill contraction, fp8 keys)."""
    qdt = _check_q(q_idx, q_scale)
    _check(w, "w", BF16)
    _check(k_idx, "k_idx", KEYS, 2)
    _check(k_scale, "k_scale", (torch.float32,), 1)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    _check(cu_q, "cu_q", (torch.int32,), 1)
    T, H_I, d_I = q_idx.shape
    B = _check_desc(ctx_len, cu_ctx, cu_q, T)
    _check_w(w, T, H_I)
    _check_keys(k_idx, k_scale, d_I)
    max_ctx = _host_max(ctx_len, max_ctx)
    if cu_q is not None:
        max_q = _host_max_q(cu_q, max_q)
    if scores is None:
        scores = torch.empty(T, max_ctx, dtype=torch.float32, device=q_idx.device)
    _check(scores, "scores", (torch.float32,), 2)
    if scores.shape[0] != T or scores.shape[1] < max_ctx:
        raise ValueError(f"scores: shape {tuple(scores.shape)}, need ({T}, >= {max_ctx})")
    if w_ld is None:
        w_ld = 0 if w.dim() == 1 else w.shape[-1]
    _call("dsa_index_scores", _p(q_idx), qdt, _p(q_scale), _p(w), w_ld, _p(k_idx),
          _key_dtype(k_idx), _p(k_scale), H_I, d_I, _p(cu_q), _p(ctx_len), _p(cu_ctx), B, T,
          max_q or 1, max_ctx, _p(scores), scores.stride(0), _stream(stream))
    return scores


def dsa_cache_append(ctx_len, cu_ctx, k_idx_cache=None, k_idx_new=None, k_scale_cache=None,
                     k_cache=None, k_new=None, v_cache=None, v_new=None, cu_q=None, stream=None):
    """Write new tokens' rows into the caches at their positions (query row t
    of the descriptor -> cache row cu_ctx[b] + p_t): the indexer key (bf16, or
    E4M3FN codes plus a per-token fp32 scale for an fp8 cache) and the K / V
    rows.  Any of the *_new tensors may be None."""
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    _check(cu_q, "cu_q", (torch.int32,), 1)
    _check(k_idx_new, "k_idx_new", BF16, 2)
    _check(k_idx_cache, "k_idx_cache", KEYS, 2)
    _check(k_scale_cache, "k_scale_cache", (torch.float32,), 1)
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check(t, n, BF16, 2)
    news = [t for t in (k_idx_new, k_new, v_new) if t is not None]
    if not news:
        return
    T = news[0].shape[0]
    B = _check_desc(ctx_len, cu_ctx, cu_q, T)
    d_I, D, kdt = 0, 0, DSA_KEY_BF16
    if k_idx_new is not None:
        if k_idx_cache is None:
            raise ValueError("k_idx_new needs k_idx_cache")
        d_I = k_idx_new.shape[1]
        _check_keys(k_idx_cache, k_scale_cache, d_I)
        kdt = _key_dtype(k_idx_cache)
    for n, new, cache in (("k", k_new, k_cache), ("v", v_new, v_cache)):
        if new is not None:
            if cache is None:
                raise ValueError(f"{n}_new needs {n}_cache")
            if new.shape[0] != T or cache.shape[1] != new.shape[1]:
                raise ValueError(f"{n}_new {tuple(new.shape)} does not fit {n}_cache "
                                 f"{tuple(cache.shape)} with {T} rows")
            D = new.shape[1]
    _call("dsa_cache_append", _p(k_idx_new), d_I, _p(k_new), _p(v_new), D, _p(cu_q), _p(ctx_len),
          _p(cu_ctx), B, T, _p(k_idx_cache), kdt, _p(k_scale_cache), _p(k_cache), _p(v_cache),
          _stream(stream))


def dsa_topk(scores, K, ctx_len, cu_q=None, max_q=None, max_ctx=None, idx=None, stream=None):
    """Exact Top-K positions per row, ascending, -1 padded: int32 [T, K]."""
    _check(scores, "scores", (torch.float32,), 2)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_q, "cu_q", (torch.int32,), 1)
    T = scores.shape[0]
    B = _check_desc(ctx_len, None, cu_q, T)
    max_ctx = _host_max(ctx_len, max_ctx)
    if scores.shape[1] < max_ctx:
        raise ValueError(f"scores: {scores.shape[1]} columns < max_ctx {max_ctx}")
    if cu_q is not None:
        max_q = _host_max_q(cu_q, max_q)
    if idx is None:
        idx = torch.empty(T, K, dtype=torch.int32, device=scores.device)
    _check(idx, "idx", (torch.int32,), 2)
    _shape(idx, "idx", (T, K))
    nbytes = load().dsa_topk_workspace_size(B, T, max_ctx, K)
    ws = _workspace(nbytes, scores.device)
    _call("dsa_topk", _p(scores), scores.stride(0), _p(cu_q), _p(ctx_len), B, T, max_q or 1,
          max_ctx, K, _p(idx), _p(ws), ws.numel(), _stream(stream))
    _keep_for(stream, ws, idx)
    return idx


def dsa_sparse_attn(q, k_cache, v_cache, idx, ctx_len, cu_ctx, window=0, gate=None, sm_scale=0.0,
                    cu_q=None, max_q=None, max_ctx=None, out=None, lse=None, stream=None):
    """Gated sparse attention; returns out bf16 [T, Hq, D] (and fills lse if given)."""
    _check(q, "q", BF16, 3)
    _check(k_cache, "k_cache", BF16, 2)
    _check(v_cache, "v_cache", BF16, 2)
    _check(idx, "idx", (torch.int32,), 2)
    _check(gate, "gate", BF16)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    _check(cu_q, "cu_q", (torch.int32,), 1)
    _check(lse, "lse", (torch.float32,), 2)
    T, Hq, D = q.shape
    B = _check_desc(ctx_len, cu_ctx, cu_q, T)
    _shape(v_cache, "v_cache", tuple(k_cache.shape))
    if k_cache.shape[1] != D:
        raise ValueError(f"k_cache: rows of {k_cache.shape[1]}, expected {D}")
    K = 0 if idx is None else idx.shape[1]
    if idx is not None:
        _shape(idx, "idx", (T, K))
    gs = _gate_stride(gate, T, Hq, D)
    _shape(lse, "lse", (T, Hq))
    max_ctx = _host_max(ctx_len, max_ctx)
    if cu_q is not None:
        max_q = _host_max_q(cu_q, max_q)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", BF16, 3)
    _shape(out, "out", (T, Hq, D))
    nbytes = load().dsa_sparse_attn_workspace_size(B, T, K, window, Hq, D)
    ws = _workspace(nbytes, q.device)
    _call("dsa_sparse_attn", _p(q), _p(k_cache), _p(v_cache), _p(idx), K, window, _p(gate), gs,
          float(sm_scale), Hq, D, _p(cu_q), _p(ctx_len), _p(cu_ctx), B, T, max_q or 1, max_ctx,
          _p(out), _p(lse), _p(ws), ws.numel(), _stream(stream))
    _keep_for(stream, ws, out)
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
    _check(gate, "gate", BF16)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    _check(out, "out", BF16, 3)
    T, Hq, D = q.shape
    B = _check_desc(ctx_len, cu_ctx, None, T)
    K = 0 if idx is None else idx.shape[1]
    if idx is not None:
        _shape(idx, "idx", (T, K))
    gs = _gate_stride(gate, T, Hq, D)
    _shape(out, "out", (T, Hq, D))
    nbytes = load().dsa_sparse_attn_workspace_size(B, T, K, window, Hq, D)
    if ws is None:
        ws = _workspace(nbytes, q.device)
    if ws.numel() < nbytes:
        raise ValueError(f"ws: {ws.numel()} bytes < {nbytes}")
    fn = load().dsa_sparse_attn
    args = (_p(q), _p(k_cache), _p(v_cache), _p(idx), K, window, _p(gate), gs, float(sm_scale),
            Hq, D, None, _p(ctx_len), _p(cu_ctx), B, T, 1, int(max_ctx), _p(out), None, _p(ws),
            ws.numel(), _stream(stream))

    def call():
        st = fn(*args)
        if st != 0:
            raise DSAError("dsa_sparse_attn", st, dsa_last_error())
    call.workspace = ws
    return call


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = None if t is None else t.data_ptr()
    return arr


def prepare_swa_decode_layers(qs, k_caches, v_caches, ctx_len, cu_ctx, max_ctx, outs, window,
                              gates=None, sm_scale=0.0, stream=None):
    """Marshal one dsa_swa_decode_layers call (all sliding-window layers of a
    decode step in one launch); returns a no-argument callable that re-issues
    it.  qs, k_caches, v_caches, outs (and gates, if given): one tensor per
    layer, kept alive and unchanged in shape while the callable is used."""
    n = len(qs)
    if not (len(k_caches) == len(v_caches) == len(outs) == n) or (gates and len(gates) != n):
        raise ValueError("one q, k_cache, v_cache, out (and gate) per layer")
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    B = _check_desc(ctx_len, cu_ctx, None, qs[0].shape[0])
    T, Hq, D = qs[0].shape
    gs = 1
    for i in range(n):
        _check(qs[i], "q", BF16, 3)
        _shape(qs[i], "q", (T, Hq, D))
        _check(k_caches[i], "k_cache", BF16, 2)
        _check(v_caches[i], "v_cache", BF16, 2)
        _shape(v_caches[i], "v_cache", tuple(k_caches[i].shape))
        if k_caches[i].shape[1] != D:
            raise ValueError(f"k_cache: rows of {k_caches[i].shape[1]}, expected {D}")
        _check(outs[i], "out", BF16, 3)
        _shape(outs[i], "out", (T, Hq, D))
        if gates and gates[i] is not None:
            _check(gates[i], "gate", BF16)
            gs = _gate_stride(gates[i], T, Hq, D)
    arrays = [_ptr_array(x) for x in (qs, k_caches, v_caches)]
    garr = _ptr_array(gates) if gates else None
    oarr = _ptr_array(outs)
    fn = load().dsa_swa_decode_layers
    args = (n, arrays[0], arrays[1], arrays[2], garr, gs, int(window), float(sm_scale), Hq, D,
            _p(ctx_len), _p(cu_ctx), B, int(max_ctx), oarr, _stream(stream))

    def call():
        st = fn(*args)
        if st != 0:
            raise DSAError("dsa_swa_decode_layers", st, dsa_last_error())
    call.keep = (arrays, garr, oarr)
    return call


def dsa_swa_decode_layers(qs, k_caches, v_caches, ctx_len, cu_ctx, window, outs=None, gates=None,
                          max_ctx=None, sm_scale=0.0, stream=None):
    """All sliding-window layers of a decode step in one launch; returns the
    list of per-layer outputs bf16 [B, Hq, D]."""
    if outs is None:
        outs = [torch.empty_like(q) for q in qs]
    max_ctx = _host_max(ctx_len, max_ctx)
    prepare_swa_decode_layers(qs, k_caches, v_caches, ctx_len, cu_ctx, max_ctx, outs, window,
                              gates=gates, sm_scale=sm_scale, stream=stream)()
    return outs


def dsa_layer_decode_workspace_size(B, max_ctx, K, Hq, D) -> int:
    return int(load().dsa_layer_decode_workspace_size(B, max_ctx, K, Hq, D))


def _layer_checks(q_idx, w, k_idx, k_scale, q, k_cache, v_cache, gate, ctx_len, cu_ctx, cu_q,
                  idx_out, K, q_dtypes=BF16):
    _check(q_idx, "q_idx", q_dtypes, 3)
    _check(w, "w", BF16)
    _check(k_idx, "k_idx", KEYS, 2)
    _check(k_scale, "k_scale", (torch.float32,), 1)
    _check(q, "q", BF16, 3)
    _check(k_cache, "k_cache", BF16, 2)
    _check(v_cache, "v_cache", BF16, 2)
    _check(gate, "gate", BF16)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_ctx, "cu_ctx", (torch.int64,), 1)
    _check(cu_q, "cu_q", (torch.int32,), 1)
    _check(idx_out, "idx_out", (torch.int32,), 2)
    T, H_I, d_I = q_idx.shape
    Tq, Hq, D = q.shape
    if Tq != T:
        raise ValueError(f"q has {Tq} rows, q_idx {T}")
    B = _check_desc(ctx_len, cu_ctx, cu_q, T)
    _check_w(w, T, H_I)
    _check_keys(k_idx, k_scale, d_I)
    _shape(v_cache, "v_cache", tuple(k_cache.shape))
    if k_cache.shape[1] != D:
        raise ValueError(f"k_cache: rows of {k_cache.shape[1]}, expected {D}")
    gs = _gate_stride(gate, T, Hq, D)
    _shape(idx_out, "idx_out", (T, K))
    return B, T, H_I, d_I, Hq, D, gs


def dsa_layer_decode(q_idx, w, k_idx, k_scale, q, k_cache, v_cache, gate, K, ctx_len, cu_ctx,
                     max_ctx=None, sm_scale=0.0, out=None, idx_out=None, ws=None, w_ld=None,
                     stream=None):
    """Whole layer for one new query per sequence; returns out bf16 [B, Hq, D].
    gate: [B, Hq, D] (elementwise), [B, Hq] (one per head) or None."""
    B, T, H_I, d_I, Hq, D, gs = _layer_checks(q_idx, w, k_idx, k_scale, q, k_cache, v_cache,
                                              gate, ctx_len, cu_ctx, None, idx_out, K)
    max_ctx = _host_max(ctx_len, max_ctx)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", BF16, 3)
    _shape(out, "out", (T, Hq, D))
    own_ws = ws is None
    if own_ws:
        ws = _workspace(dsa_layer_decode_workspace_size(B, max_ctx, K, Hq, D), q.device)
    if w_ld is None:
        w_ld = 0 if w.dim() == 1 else w.shape[-1]
    _call("dsa_layer_decode", _p(q_idx), _p(w), w_ld, _p(k_idx), _key_dtype(k_idx), _p(k_scale),
          H_I, d_I, _p(q), _p(k_cache), _p(v_cache), _p(gate), gs, float(sm_scale), Hq, D, K,
          _p(ctx_len), _p(cu_ctx), B, max_ctx, _p(out), _p(idx_out), _p(ws), ws.numel(),
          _stream(stream))
    _keep_for(stream, ws if own_ws else None, out)
    return out


def dsa_layer_decode_append(q_idx, w, k_idx, k_scale, q, k_cache, v_cache, gate, K, ctx_len,
                            cu_ctx, k_idx_new, k_new=None, v_new=None, max_ctx=None, sm_scale=0.0,
                            out=None, idx_out=None, ws=None, w_ld=None, stream=None):
    """Decode layer with each sequence's new token appended to the caches first
    (row cu_ctx[b] + ctx_len[b] - 1): k_idx_new bf16 [B, d_I] (quantised for an
    fp8 key cache), k_new / v_new bf16 [B, D].  The caches are written."""
    B, T, H_I, d_I, Hq, D, gs = _layer_checks(q_idx, w, k_idx, k_scale, q, k_cache, v_cache,
                                              gate, ctx_len, cu_ctx, None, idx_out, K)
    _check(k_idx_new, "k_idx_new", BF16, 2)
    _shape(k_idx_new, "k_idx_new", (B, d_I))
    _check(k_new, "k_new", BF16, 2)
    _check(v_new, "v_new", BF16, 2)
    _shape(k_new, "k_new", (B, D))
    _shape(v_new, "v_new", (B, D))
    max_ctx = _host_max(ctx_len, max_ctx)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", BF16, 3)
    _shape(out, "out", (T, Hq, D))
    own_ws = ws is None
    if own_ws:
        ws = _workspace(dsa_layer_decode_workspace_size(B, max_ctx, K, Hq, D), q.device)
    if w_ld is None:
        w_ld = 0 if w.dim() == 1 else w.shape[-1]
    _call("dsa_layer_decode_append", _p(q_idx), _p(w), w_ld, _p(k_idx), _key_dtype(k_idx),
          _p(k_scale), H_I, d_I, _p(q), _p(k_cache), _p(v_cache), _p(gate), gs, float(sm_scale),
          Hq, D, K, _p(ctx_len), _p(cu_ctx), B, max_ctx, _p(k_idx_new), _p(k_new), _p(v_new),
          _p(out), _p(idx_out), _p(ws), ws.numel(), _stream(stream))
    _keep_for(stream, ws if own_ws else None, out)
    return out


def prepare_layer_decode(q_idx, w, k_idx, k_scale, q, k_cache, v_cache, gate, K, ctx_len, cu_ctx,
                         max_ctx, out, ws, sm_scale=0.0, idx_out=None, w_ld=None, stream=None):
    """Marshal one dsa_layer_decode call once; returns a no-argument callable
    that re-issues it (one ctypes call, no per-call argument checks).  The
    tensors must stay alive and unchanged in shape while the callable is used."""
    B, T, H_I, d_I, Hq, D, gs = _layer_checks(q_idx, w, k_idx, k_scale, q, k_cache, v_cache,
                                              gate, ctx_len, cu_ctx, None, idx_out, K)
    _check(out, "out", BF16, 3)
    _shape(out, "out", (T, Hq, D))
    need = dsa_layer_decode_workspace_size(B, int(max_ctx), K, Hq, D)
    if ws.numel() < need:
        raise ValueError(f"ws: {ws.numel()} bytes < {need}")
    if w_ld is None:
        w_ld = 0 if w.dim() == 1 else w.shape[-1]
    fn = load().dsa_layer_decode
    args = (_p(q_idx), _p(w), w_ld, _p(k_idx), _key_dtype(k_idx), _p(k_scale), H_I, d_I, _p(q),
            _p(k_cache), _p(v_cache), _p(gate), gs, float(sm_scale), Hq, D, K, _p(ctx_len),
            _p(cu_ctx), B, int(max_ctx), _p(out), _p(idx_out), _p(ws), ws.numel(),
            _stream(stream))

    def call():
        st = fn(*args)
        if st != 0:
            raise DSAError("dsa_layer_decode", st, dsa_last_error())
    return call


def dsa_layer_decode_noalloc(q_idx, w, k_idx, k_scale, q, k_cache, v_cache, gate, K, ctx_len,
                             cu_ctx, max_ctx, out, idx_out=None, sm_scale=0.0, w_ld=None,
                             stream=None):
    """dsa_layer_decode without a workspace argument: the library's fixed
    per-GPU scratch array serves as workspace and nothing is allocated (the
    caller passes `out` and `max_ctx`).  Calls overlapping on one GPU race."""
    B, T, H_I, d_I, Hq, D, gs = _layer_checks(q_idx, w, k_idx, k_scale, q, k_cache, v_cache,
                                              gate, ctx_len, cu_ctx, None, idx_out, K)
    _check(out, "out", BF16, 3)
    _shape(out, "out", (T, Hq, D))
    if w_ld is None:
        w_ld = 0 if w.dim() == 1 else w.shape[-1]
    _call("dsa_layer_decode_noalloc", _p(q_idx), _p(w), w_ld, _p(k_idx), _key_dtype(k_idx),
          _p(k_scale), H_I, d_I, _p(q), _p(k_cache), _p(v_cache), _p(gate), gs, float(sm_scale),
          Hq, D, K, _p(ctx_len), _p(cu_ctx), B, int(max_ctx), _p(out), _p(idx_out),
          _stream(stream))
    return out


def layer_scores(ws, rows, max_ctx):
    """View of the fp32 indexer scores a layer call left at the start of its
    workspace `ws` (uint8 tensor): [rows, ld] with ld = max_ctx rounded up to
    a multiple of 64 (the documented workspace contract of dsa_layer_decode
    and of a one-pass dsa_layer_prefill)."""
    ld = (int(max_ctx) + 63) // 64 * 64
    return ws[:rows * ld * 4].view(torch.float32).view(rows, ld)


def dsa_set_indexer_events(start, stop):
    """Record the caller's HIP events (raw hipEvent_t handles as ints, or
    None, None) around the indexer launch of later dsa_layer_decode calls
    on this thread."""
    _call("dsa_set_indexer_events", start, stop)


def dsa_set_topk_counters(counters):
    """Count, per Top-K row on this thread, the path that produced it into a
    caller-owned uint32 [6] device tensor (certified union, exact fallback,
    direct, row sweeps, of those the sampled-threshold ones, and failed
    unions resolved by one collection sweep); None stops counting."""
    if counters is not None:
        assert counters.dtype == torch.int32
        assert counters.is_cuda and counters.numel() >= 6 and counters.is_contiguous()
    _call("dsa_set_topk_counters", None if counters is None else counters.data_ptr())


def _check_counters(counters, n):
    _check(counters, "counters", (torch.int32,), 1)
    if counters.numel() < n:
        raise ValueError(f"counters: need {n} entries, got {counters.numel()}")


def dsa_check_index_rows(idx, ctx_len, cu_q=None, full=True, counters=None, stream=None):
    """Debug check of index rows idx [T, K] (int32) against each row's query
    position: adds into counters (int32 [4] on the device; a zeroed one is
    made when None) the entries outside [0, p] other than -1, with `full`
    the order breaks and the rows whose count is not min(K, p + 1), and the
    rows checked.  Returns the counters tensor (not synchronised)."""
    _check(idx, "idx", (torch.int32,), 2)
    _check(ctx_len, "ctx_len", (torch.int32,), 1)
    _check(cu_q, "cu_q", (torch.int32,), 1)
    T, K = idx.shape
    B = ctx_len.numel() if cu_q is None else cu_q.numel() - 1
    if counters is None:
        counters = torch.zeros(4, dtype=torch.int32, device=idx.device)
    _check_counters(counters, 4)
    _call("dsa_check_index_rows", _p(idx), K, _p(cu_q), _p(ctx_len), B, T, 1 if full else 0,
          _p(counters), _stream(stream))
    _keep_for(stream, counters)
    return counters


def dsa_set_index_checks(counters):
    """Run the index-row check after every selection (and on the caller's rows
    before dsa_sparse_attn gathers with them) on this thread, adding into a
    caller-owned int32 [4] device tensor; None stops."""
    if counters is not None:
        _check_counters(counters, 4)
    _call("dsa_set_index_checks", None if counters is None else counters.data_ptr())


def dsa_layer_prefill_workspace_size(B, T, max_ctx, K, Hq, D) -> int:
    """Workspace bytes that run all T query rows in one pass."""
    return int(load().dsa_layer_prefill_workspace_size(B, T, max_ctx, K, Hq, D))


def dsa_layer_prefill_min_workspace_size(B, max_ctx, K, Hq, D) -> int:
    """Least workspace bytes a prefill call accepts (rows then run in sub-chunks)."""
    return int(load().dsa_layer_prefill_min_workspace_size(B, max_ctx, K, Hq, D))


def dsa_layer_prefill(q_idx, w, k_idx, k_scale, q, k_cache, v_cache, gate, K, cu_q, ctx_len,
                      cu_ctx, max_q=None, max_ctx=None, sm_scale=0.0, out=None, idx_out=None,
                      ws=None, w_ld=None, stream=None, q_scale=None):
    """Whole layer for a chunk of new queries per sequence; returns out bf16 [T, Hq, D].
    A caller workspace smaller than the one-pass size (but at least the
    minimum) makes the library run the rows in sub-chunks.  q_idx is bf16, or
    E4M3FN with q_scale [T, H_I] (fp8 MFMA indexer; needs fp8 keys)."""
    qdt = _check_q(q_idx, q_scale)
    B, T, H_I, d_I, Hq, D, gs = _layer_checks(q_idx, w, k_idx, k_scale, q, k_cache, v_cache,
                                              gate, ctx_len, cu_ctx, cu_q, idx_out, K, KEYS)
    max_ctx = _host_max(ctx_len, max_ctx)
    max_q = _host_max_q(cu_q, max_q)
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", BF16, 3)
    _shape(out, "out", (T, Hq, D))
    own_ws = ws is None
    if own_ws:
        ws = _workspace(dsa_layer_prefill_workspace_size(B, T, max_ctx, K, Hq, D), q.device)
    if w_ld is None:
        w_ld = 0 if w.dim() == 1 else w.shape[-1]
    _call("dsa_layer_prefill", _p(q_idx), qdt, _p(q_scale), _p(w), w_ld, _p(k_idx),
          _key_dtype(k_idx),
          _p(k_scale), H_I, d_I, _p(q), _p(k_cache), _p(v_cache), _p(gate), gs, float(sm_scale),
          Hq, D, K, _p(cu_q), _p(ctx_len), _p(cu_ctx), B, T, max_q, max_ctx, _p(out), _p(idx_out),
          _p(ws), ws.numel(), _stream(stream))
    _keep_for(stream, ws if own_ws else None, out)
    return out
