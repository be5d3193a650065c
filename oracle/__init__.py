"""oracle -- ctypes binding of the plain fp64 CPU oracle in dsa_oracle.c.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke()
and by the CPU-baseline leg of bench.py.  The product library
(long_context_sparse_dsa_amd) never imports, loads or calls anything here,
and this package shares no code with it.

What each function computes is documented in dsa_oracle.c next to the C
function it wraps (Indexer score, Top-K select, gated sparse attention,
whole layer), with the passages of the pages each one follows.

Inputs are numpy arrays or CPU torch tensors; bf16 tensors are passed by
their bit patterns (uint16), fp8 e4m3fn tensors by their codes (uint8).
Results are float64 numpy arrays (indices: int32).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libdsa_oracle.so")

KEY_BF16 = 0
KEY_FP8_E4M3 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile dsa_oracle.c with gcc into oracle/libdsa_oracle.so."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-pthread", "-Wall", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f64.restype = D
        lib.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_to_f64.restype = D
        lib.orc_quantize_e4m3_rows.argtypes = [P, L, I, P, P]
        lib.orc_quantize_e4m3_rows.restype = I
        lib.orc_index_scores.argtypes = [P, I, P, P, L, P, I, P, I, I, P, P, P, I, P, L, I]
        lib.orc_index_scores.restype = I
        lib.orc_topk_f64.argtypes = [P, L, P, P, I, I, P, I]
        lib.orc_topk_f64.restype = I
        lib.orc_topk_f32.argtypes = [P, L, P, P, I, I, P, I]
        lib.orc_topk_f32.restype = I
        lib.orc_sparse_attn.argtypes = [P, P, P, P, I, I, P, D, I, I, P, P, P, I, P, P, I]
        lib.orc_sparse_attn.restype = I
        lib.orc_layer.argtypes = [P, P, L, P, I, P, I, I, P, P, P, P, D, I, I, I, P, P, P, I,
                                  P, P, P, P, L, I]
        lib.orc_layer.restype = I
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
               else (os.cpu_count() or 1))


# ---------------------------------------------------------------------------
# Marshalling helpers (no arithmetic of the method here).
# ---------------------------------------------------------------------------

def _np(x, dtype=None):
    """Contiguous numpy view of x; torch bf16 -> uint16 bits, fp8 -> uint8."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16).numpy().view(np.uint16)
            elif x.dtype == getattr(torch, "float8_e4m3fn", None):
                x = x.view(torch.uint8).numpy()
            else:
                x = x.numpy()
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if dtype is not None and x.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {x.dtype}")
    return x


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _desc(cu_q, ctx_len, cu_ctx, B):
    ctx_len = _np(ctx_len).astype(np.int32)
    B = int(ctx_len.shape[0]) if B is None else B
    if cu_q is None:
        cu_q = np.arange(B + 1, dtype=np.int32)
    cu_q = _np(cu_q).astype(np.int32)
    if cu_ctx is None:
        cu_ctx = np.concatenate([[0], np.cumsum(ctx_len.astype(np.int64))]).astype(np.int64)
    cu_ctx = _np(cu_ctx).astype(np.int64)
    if cu_q.shape != (B + 1,) or cu_ctx.shape != (B + 1,):
        raise ValueError("batch descriptor: cu_q and cu_ctx need B+1 entries")
    nq = np.diff(cu_q)
    if np.any(nq < 0) or np.any(nq > ctx_len):
        raise ValueError("batch descriptor: 0 <= n_q <= ctx_len per sequence")
    return cu_q, ctx_len, cu_ctx, B


def _keys(k_idx):
    k = _np(k_idx)
    if k.dtype == np.uint16:
        return k, KEY_BF16
    if k.dtype == np.uint8:
        return k, KEY_FP8_E4M3
    raise TypeError("indexer keys must be bf16 (uint16 bits) or fp8 e4m3fn (uint8 codes)")


# ---------------------------------------------------------------------------
# Public oracle functions.
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    lib = _load()
    b = _np(bits).astype(np.uint16).ravel()
    return np.array([lib.orc_bf16_to_f64(int(v)) for v in b], dtype=np.float64)


def e4m3_to_f64(codes) -> np.ndarray:
    lib = _load()
    c = _np(codes).astype(np.uint8).ravel()
    return np.array([lib.orc_e4m3_to_f64(int(v)) for v in c], dtype=np.float64)


def quantize_e4m3_rows(k_rows):
    """Cache-append quantisation of bf16 key rows [n, d]: returns (codes uint8
    [n, d] (E4M3FN), scales float32 [n]) with per-row absolute-maximum
    scaling (see dsa_oracle.c)."""
    lib = _load()
    k = _np(k_rows, np.uint16)
    n, d = k.shape
    codes = np.zeros((n, d), dtype=np.uint8)
    scales = np.zeros(n, dtype=np.float32)
    lib.orc_quantize_e4m3_rows(_ptr(k), n, d, _ptr(codes), _ptr(scales))
    return codes, scales


def index_scores(q_idx, w, k_idx, k_scale=None, ctx_len=None, cu_q=None, cu_ctx=None,
                 w_ld=None, ld=None, nthreads=None, q_scale=None):
    """Indexer scores [T, ld] in fp64; entries j > p_t are NaN.  Query heads
    are bf16, or E4M3FN codes with q_scale fp32 [T, H] (one per query and
    head)."""
    lib = _load()
    q, qdt = _keys(q_idx)
    if (qdt == KEY_FP8_E4M3) != (q_scale is not None):
        raise ValueError("E4M3FN query heads take a q_scale, bf16 ones none")
    qs = None if q_scale is None else _np(q_scale).astype(np.float32)
    T, H, d = q.shape
    if qs is not None and qs.shape != (T, H):
        raise ValueError("q_scale must be [T, H]")
    wv = _np(w, np.uint16)
    if w_ld is None:
        w_ld = 0 if wv.ndim == 1 else wv.shape[-1]
    k, kdt = _keys(k_idx)
    ks = None if k_scale is None else _np(k_scale).astype(np.float32)
    cu_q, ctx_len, cu_ctx, B = _desc(cu_q, ctx_len, cu_ctx, None)
    if ld is None:
        ld = int(ctx_len.max())
    out = np.full((T, ld), np.nan, dtype=np.float64)
    lib.orc_index_scores(_ptr(q), qdt, _ptr(qs), _ptr(wv), w_ld, _ptr(k), kdt, _ptr(ks), H, d,
                         _ptr(cu_q), _ptr(ctx_len), _ptr(cu_ctx), B, _ptr(out), ld,
                         nthreads or default_threads())
    return out


def topk(scores, K, ctx_len, cu_q=None, nthreads=None):
    """Exact Top-K per row; fp64 scores -> Mode E, fp32 scores -> Mode T."""
    lib = _load()
    s = _np(scores)
    cu_q, ctx_len, _, B = _desc(cu_q, ctx_len, None, None)
    T, ld = s.shape
    idx = np.zeros((T, K), dtype=np.int32)
    fn = {np.dtype(np.float64): lib.orc_topk_f64, np.dtype(np.float32): lib.orc_topk_f32}
    if s.dtype not in fn:
        raise TypeError("scores must be float32 or float64")
    fn[s.dtype](_ptr(s), ld, _ptr(cu_q), _ptr(ctx_len), B, K, _ptr(idx),
                nthreads or default_threads())
    return idx


def sparse_attn(q, k_cache, v_cache, idx=None, window=0, gate=None, sm_scale=0.0,
                ctx_len=None, cu_q=None, cu_ctx=None, nthreads=None):
    """Gated sparse attention; returns (out [T,Hq,D] fp64, lse [T,Hq] fp64)."""
    lib = _load()
    qv = _np(q, np.uint16)
    T, Hq, D = qv.shape
    kc = _np(k_cache, np.uint16)
    vc = _np(v_cache, np.uint16)
    iv = None if idx is None else _np(idx).astype(np.int32)
    K = 0 if iv is None else iv.shape[1]
    g = None if gate is None else _np(gate, np.uint16)
    cu_q, ctx_len, cu_ctx, B = _desc(cu_q, ctx_len, cu_ctx, None)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.zeros((T, Hq), dtype=np.float64)
    lib.orc_sparse_attn(_ptr(qv), _ptr(kc), _ptr(vc), _ptr(iv), K, window, _ptr(g),
                        float(sm_scale), Hq, D, _ptr(cu_q), _ptr(ctx_len), _ptr(cu_ctx), B,
                        _ptr(out), _ptr(lse), nthreads or default_threads())
    return out, lse


def layer(q_idx, w, k_idx, k_scale, q, k_cache, v_cache, gate, K, ctx_len, cu_q=None,
          cu_ctx=None, sm_scale=0.0, w_ld=None, nthreads=None):
    """Whole layer; returns dict(out, lse, scores, idx) (all fp64 / int32)."""
    lib = _load()
    qi = _np(q_idx, np.uint16)
    T, H, d = qi.shape
    wv = _np(w, np.uint16)
    if w_ld is None:
        w_ld = 0 if wv.ndim == 1 else wv.shape[-1]
    k, kdt = _keys(k_idx)
    ks = None if k_scale is None else _np(k_scale).astype(np.float32)
    qv = _np(q, np.uint16)
    _, Hq, D = qv.shape
    kc = _np(k_cache, np.uint16)
    vc = _np(v_cache, np.uint16)
    g = None if gate is None else _np(gate, np.uint16)
    cu_q, ctx_len, cu_ctx, B = _desc(cu_q, ctx_len, cu_ctx, None)
    ld = int(ctx_len.max())
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.zeros((T, Hq), dtype=np.float64)
    scores = np.full((T, ld), np.nan, dtype=np.float64)
    idx = np.zeros((T, K), dtype=np.int32)
    lib.orc_layer(_ptr(qi), _ptr(wv), w_ld, _ptr(k), kdt, _ptr(ks), H, d, _ptr(qv), _ptr(kc),
                  _ptr(vc), _ptr(g), float(sm_scale), Hq, D, K, _ptr(cu_q), _ptr(ctx_len),
                  _ptr(cu_ctx), B, _ptr(out), _ptr(lse), _ptr(scores), _ptr(idx), ld,
                  nthreads or default_threads())
    return {"out": out, "lse": lse, "scores": scores, "idx": idx}
