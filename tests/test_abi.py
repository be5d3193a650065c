"""The C ABI of libdsa.so on a host without a GPU: it loads, exports every
entry point include/dsa.h declares, sizes workspaces, and rejects invalid
arguments during host-side validation (before any HIP call)."""
import ctypes
import os
import re

import pytest

import long_context_sparse_dsa_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: validation fails first
FAKE_MIS = ctypes.c_void_p(0x10004)  # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return dsa.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dsa.EXPORTS)


def test_version_and_error_strings(lib):
    assert "gfx950" in dsa.dsa_version()
    assert isinstance(dsa.dsa_last_error(), str)


def test_workspace_sizes_are_sane(lib):
    small = lib.dsa_layer_decode_workspace_size(1, 4096, 256, 8, 64)
    big = lib.dsa_layer_decode_workspace_size(1, 131072, 2048, 64, 128)
    assert 0 < small < big
    # scores (fp32 per position) dominate the decode workspace
    assert big >= 131072 * 4
    assert lib.dsa_topk_workspace_size(1, 8, 100000, 2048) > 0
    assert lib.dsa_topk_workspace_size(1, 0, 100000, 2048) == 0
    assert lib.dsa_sparse_attn_workspace_size(1, 1, 2048, 0, 64, 128) > 0
    assert lib.dsa_sparse_attn_workspace_size(1, 8192, 2048, 0, 64, 128) == 0   # no split
    pre = lib.dsa_layer_prefill_workspace_size(1, 8192, 139264, 2048, 64, 128)
    assert pre >= 8192 * 139264 * 4


def _idx_scores(lib, **kw):
    a = dict(q=FAKE, qdt=0, qs=None, w=FAKE, w_ld=32, k=FAKE, kdt=0, ks=None, H=32, d=128, cu_q=None,
             ctx=FAKE, cu_ctx=FAKE, B=1, T=1, max_q=1, max_ctx=1000, scores=FAKE, ld=1000)
    a.update(kw)
    return lib.dsa_index_scores(a["q"], a["qdt"], a["qs"], a["w"], a["w_ld"], a["k"], a["kdt"],
                                a["ks"], a["H"], a["d"], a["cu_q"], a["ctx"], a["cu_ctx"], a["B"],
                                a["T"], a["max_q"], a["max_ctx"], a["scores"], a["ld"], None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(q=None), 1, "q_idx"),
    (dict(k=FAKE_MIS), 1, "aligned"),
    (dict(H=8), 2, "indexer shape"),
    (dict(d=96), 2, "indexer shape"),
    (dict(kdt=1), 1, "k_scale"),
    (dict(ks=FAKE), 1, "bf16 keys"),
    (dict(kdt=7), 1, "k_dtype"),
    (dict(ld=999), 1, "ld"),
    (dict(T=2), 1, "T (2) must equal B"),
    (dict(B=0), 1, "B must be"),
    (dict(w_ld=5), 1, "w_ld"),
    (dict(cu_q=FAKE, max_q=0), 1, "max_q"),
    (dict(ctx=None), 1, "ctx_len"),
    (dict(qdt=1), 1, "q_scale"),
    (dict(qdt=1, qs=FAKE), 2, "fp8 key cache"),
    (dict(qdt=1, qs=FAKE, kdt=1, ks=FAKE), 2, "prefill contraction"),
    (dict(qs=FAKE), 1, "bf16 query heads"),
    (dict(qdt=3), 1, "q_dtype"),
])
def test_index_scores_validation(lib, kw, code, frag):
    assert _idx_scores(lib, **kw) == code
    assert frag in dsa.dsa_last_error()


def test_topk_validation(lib):
    f = lib.dsa_topk
    assert f(FAKE, 100, None, FAKE, 1, 1, 1, 100, 0, FAKE, FAKE, 1 << 20, None) == 2
    assert "K must be" in dsa.dsa_last_error()
    assert f(FAKE, 100, None, FAKE, 1, 1, 1, 100, 5000, FAKE, FAKE, 1 << 20, None) == 2
    assert f(FAKE, 50, None, FAKE, 1, 1, 1, 100, 16, FAKE, FAKE, 1 << 20, None) == 1
    assert f(FAKE, 100, None, FAKE, 1, 1, 1, 100, 16, FAKE, FAKE, 1, None) == 3
    assert "workspace too small" in dsa.dsa_last_error()
    assert f(None, 100, None, FAKE, 1, 1, 1, 100, 16, FAKE, FAKE, 1 << 20, None) == 1


def test_sparse_attn_validation(lib):
    f = lib.dsa_sparse_attn
    # unsupported head geometry
    assert f(FAKE, FAKE, FAKE, FAKE, 16, 0, None, 1, 0.0, 32, 128, None, FAKE, FAKE, 1, 1, 1, 100,
             FAKE, None, FAKE, 1 << 20, None) == 2
    # window mode without a window
    assert f(FAKE, FAKE, FAKE, None, 0, 0, None, 1, 0.0, 64, 128, None, FAKE, FAKE, 1, 1, 1, 100,
             FAKE, None, FAKE, 1 << 20, None) == 2
    assert "window" in dsa.dsa_last_error()
    # negative scale
    assert f(FAKE, FAKE, FAKE, FAKE, 16, 0, None, 1, -1.0, 64, 128, None, FAKE, FAKE, 1, 1, 1,
             100, FAKE, None, FAKE, 1 << 20, None) == 1
    # split plan needs a workspace
    assert f(FAKE, FAKE, FAKE, FAKE, 2048, 0, None, 1, 0.0, 64, 128, None, FAKE, FAKE, 1, 1, 1,
             100000, FAKE, None, FAKE, 16, None) == 3
    # the gate's dim stride is 1 (elementwise) or 0 (one value per head)
    assert f(FAKE, FAKE, FAKE, FAKE, 16, 0, FAKE, 2, 0.0, 64, 128, None, FAKE, FAKE, 1, 1, 1, 100,
             FAKE, None, FAKE, 1 << 20, None) == 1
    assert "gate_stride_d" in dsa.dsa_last_error()


def test_layer_validation(lib):
    f = lib.dsa_layer_decode
    args = [FAKE, FAKE, 32, FAKE, 0, None, 32, 128, FAKE, FAKE, FAKE, FAKE, 1, 0.0, 64, 128,
            2048, FAKE, FAKE, 1, 131072, FAKE, None, FAKE, 16, None]
    assert f(*args) == 3
    args2 = list(args)
    args2[16] = 0   # K
    assert f(*args2) == 2
    args3 = list(args)
    args3[12] = -1  # gate_stride_d
    assert f(*args3) == 1 and "gate_stride_d" in dsa.dsa_last_error()
    g = lib.dsa_layer_prefill
    pargs = [FAKE, 0, None, FAKE, 16, FAKE, 0, None, 16, 128, FAKE, FAKE, FAKE, FAKE, 1, 0.0, 64,
             128, 2048, None, FAKE, FAKE, 1, 8192, 8192, 139264, FAKE, None, FAKE, 1 << 40, None]
    assert g(*pargs) == 1
    assert "cu_q" in dsa.dsa_last_error()
    # below the least workspace: refused before any launch, sizes in the message
    small = list(pargs)
    small[19] = FAKE
    small[29] = lib.dsa_layer_prefill_min_workspace_size(1, 139264, 2048, 64, 128) - 1
    assert g(*small) == 3
    assert "workspace too small" in dsa.dsa_last_error()


def test_prefill_workspace_sizes(lib):
    full = lib.dsa_layer_prefill_workspace_size(1, 8192, 139264, 2048, 64, 128)
    least = lib.dsa_layer_prefill_min_workspace_size(1, 139264, 2048, 64, 128)
    # one query row: its fp32 score row plus small scratch, far below one pass
    assert 139264 * 4 < least < 8 * 1024 * 1024 < full
    assert lib.dsa_layer_prefill_min_workspace_size(0, 139264, 2048, 64, 128) == 0


def test_workspace_sizes_over_a_grid_of_extreme_shapes(lib):
    """Every size function over extreme but representable shapes: no
    overflow (the sanitized build traps signed overflow), sizes grow with
    the problem, and an empty batch needs nothing."""
    prev = 0
    for max_ctx in (1, 2047, 2048, 16384, 16385, 131072, 1 << 20, 1 << 24, (1 << 31) - 1):
        d = lib.dsa_layer_decode_workspace_size(1, max_ctx, 2048, 64, 128)
        assert d >= prev and d >= 4 * max_ctx
        prev = d
        for B in (1, 7, 1024, 4096):
            for K in (1, 256, 2048, 4096):
                assert lib.dsa_layer_decode_workspace_size(B, max_ctx, K, 8, 64) > 0
                assert lib.dsa_topk_workspace_size(B, B, max_ctx, K) >= 0
                assert lib.dsa_layer_prefill_min_workspace_size(B, max_ctx, K, 64, 128) > 0
        assert lib.dsa_layer_prefill_workspace_size(1, 8192, max_ctx, 2048, 64, 128) > 0
    for T in (1, 255, 256, 8192, 1 << 20):
        assert lib.dsa_sparse_attn_workspace_size(1, T, 2048, 0, 64, 128) >= 0
        assert lib.dsa_sparse_attn_workspace_size(8, T, 0, 128, 64, 128) >= 0
    assert lib.dsa_layer_decode_workspace_size(0, 131072, 2048, 64, 128) >= 0
    assert lib.dsa_layer_decode_noalloc_max_bytes() > 0


def test_device_calls_without_a_device_report_a_hip_error(lib):
    """On a host with no GPU the library loads, validation still answers,
    and a well-formed call reports DSA_ERR_HIP instead of crashing."""
    import torch
    if torch.cuda.device_count() != 0:
        pytest.skip("a GPU is visible: this check runs only where none is")
    n = 4096
    ws_bytes = lib.dsa_layer_decode_workspace_size(1, n, 256, 8, 64)
    st = lib.dsa_layer_decode(FAKE, FAKE, 4, FAKE, 0, None, 4, 64, FAKE, FAKE, FAKE, FAKE, 1, 0.0,
                              8, 64, 256, FAKE, FAKE, 1, n, FAKE, None, FAKE, ws_bytes, None)
    assert st == 4
    assert dsa.dsa_last_error()


def test_index_check_validation(lib):
    f = lib.dsa_check_index_rows
    assert f(None, 16, None, FAKE, 1, 1, 1, FAKE, None) == 1 and "idx" in dsa.dsa_last_error()
    assert f(FAKE, 0, None, FAKE, 1, 1, 1, FAKE, None) == 1 and "K must be" in dsa.dsa_last_error()
    assert f(FAKE, 16, None, FAKE, 2, 3, 1, FAKE, None) == 1
    assert f(FAKE, 16, None, None, 1, 1, 1, FAKE, None) == 1
    assert f(FAKE, 16, None, FAKE, 1, 1, 1, FAKE_MIS, None) == 1
    assert lib.dsa_set_index_checks(None) == 0


def test_trace_ranges_load_on_demand():
    """DSA_TRACE=1 opens the roctx library on the first call that would
    enqueue work; validation and error reporting behave as without it."""
    import subprocess
    import sys
    code = ("import ctypes, long_context_sparse_dsa_amd as dsa\n"
            "lib = dsa.load()\n"
            "F = ctypes.c_void_p(0x10000)\n"
            "st = lib.dsa_topk(F, 100, None, F, 1, 1, 1, 100, 0, F, F, 1 << 20, None)\n"
            "assert st == 2, st\n"
            "assert 'K must be' in dsa.dsa_last_error()\n"
            "print('trace ok')\n")
    env = dict(os.environ, DSA_TRACE="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "trace ok" in r.stdout
