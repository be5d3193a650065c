"""Parity of the HIP library (through its C ABI) with the fp64 oracle.

Small cases compare every output element and span several tiles plus a
ragged tail; the full-size cases (the bench's 128K decode, the 1M fp8
batched decode and the 8K-query prefill chunk) compare sampled rows that
the oracle computes one by one.  Inputs come from the seeded generators in
long_context_sparse_dsa_amd.workloads.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from long_context_sparse_dsa_amd import workloads as W
from tests.parity import (ATOL_BF16, ATOL_FP8, FP8_MFMA_REL, check_index_row, check_out,
                          check_set_band, cpu, fp8_score_bound, positions)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def wl(name, ctx_lens, n_q, H_I, d_I, Hq, D, K, **kw):
    return W.Workload(name, list(ctx_lens), list(n_q), H_I, d_I, Hq, D, K, **kw)


# --------------------------------------------------------------------------
# Indexer scores
# --------------------------------------------------------------------------

def _score_tol(ref):
    scale = np.nanmax(np.abs(ref))
    return 1e-5 * scale + 1e-5 * np.abs(ref)


@pytest.mark.parametrize("H_I,d_I,key,lens", [
    (4, 64, "bf16", [4096]),
    (32, 128, "bf16", [5000]),
    (16, 128, "bf16", [300, 2049, 777]),
    (32, 128, "fp8", [3001, 1500]),
    (16, 128, "fp8", [1100]),
])
def test_index_scores_decode(dsa, H_I, d_I, key, lens):
    say(f"index_scores decode H_I={H_I} d_I={d_I} {key} lens={lens}")
    w = wl("t", lens, [1] * len(lens), H_I, d_I, 8, 64, 64, key_dtype=key, seed=11)
    inp = W.make_inputs(w)
    d = to_dev(inp)
    s = dsa.dsa_index_scores(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["ctx_len"],
                             d["cu_ctx"], max_ctx=max(lens))
    torch.cuda.synchronize()
    ref = oracle.index_scores(inp["q_idx"], inp["w"], inp["k_idx"], inp["k_scale"],
                              ctx_len=inp["ctx_len"], cu_ctx=inp["cu_ctx"])
    got = s.cpu().numpy().astype(np.float64)
    for b, L in enumerate(lens):
        err = np.abs(got[b, :L] - ref[b, :L])
        assert np.all(err <= _score_tol(ref[b, :L])), f"row {b}: max err {err.max():.3g}"


@pytest.mark.parametrize("H_I,d_I,key,lens,nq,qdt", [
    (16, 128, "bf16", [3000], [200], "bf16"),
    (32, 128, "bf16", [2500, 700], [70, 33], "bf16"),
    (4, 64, "bf16", [1200], [130], "bf16"),
    (16, 128, "fp8", [2100], [90], "bf16"),
    # fp8 query heads with per-(query, head) scales on the fp8 MFMA
    (16, 128, "fp8", [3000, 700], [200, 45], "fp8"),
    (32, 128, "fp8", [2500], [70], "fp8"),
    (4, 64, "fp8", [1200, 300], [130, 7], "fp8"),
])
def test_index_scores_prefill(dsa, H_I, d_I, key, lens, nq, qdt):
    say(f"index_scores prefill H_I={H_I} keys {key} queries {qdt} lens={lens} nq={nq}")
    w = wl("t", lens, nq, H_I, d_I, 8, 64, 64, key_dtype=key, q_dtype=qdt, seed=12)
    inp = W.make_inputs(w)
    d = to_dev(inp)
    s = torch.full((w.T, max(lens)), float("nan"), device=DEV)
    dsa.dsa_index_scores(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["ctx_len"], d["cu_ctx"],
                         cu_q=d["cu_q"], max_ctx=max(lens), scores=s, q_scale=d["q_scale"])
    torch.cuda.synchronize()
    ref = oracle.index_scores(inp["q_idx"], inp["w"], inp["k_idx"], inp["k_scale"],
                              ctx_len=inp["ctx_len"], cu_q=inp["cu_q"], cu_ctx=inp["cu_ctx"],
                              q_scale=inp["q_scale"])
    got = s.cpu().numpy().astype(np.float64)
    bound = None
    if qdt == "fp8":
        bound = fp8_score_bound(inp["q_idx"], inp["w"], inp["k_idx"], inp["k_scale"],
                                inp["q_scale"], ctx_len=inp["ctx_len"], cu_q=inp["cu_q"],
                                cu_ctx=inp["cu_ctx"])
    for t, p in enumerate(positions(lens, nq)):
        err = np.abs(got[t, :p + 1] - ref[t, :p + 1])
        if bound is None:
            tol = _score_tol(ref[t, :p + 1])
        else:
            tol = FP8_MFMA_REL * bound[t, :p + 1] + 1e-6 * np.abs(ref[t, :p + 1])
        assert np.all(err <= tol), f"row {t}: max err {err.max():.3g}"
        assert np.all(np.isnan(got[t, p + 1:])), f"row {t}: wrote past its position"


# --------------------------------------------------------------------------
# Top-K: bit-exact on identical fp32 arrays
# --------------------------------------------------------------------------

def _topk_case(kind, n, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "normal":
        return torch.randn(n, generator=g)
    if kind == "ties":
        return torch.round(torch.randn(n, generator=g) * 4) / 4
    if kind == "equal":
        return torch.full((n,), 2.5)
    if kind == "ramp":
        return torch.arange(n, dtype=torch.float32)
    if kind == "ramp_down":
        return -torch.arange(n, dtype=torch.float32)
    if kind == "zeros_signed":
        x = torch.zeros(n)
        x[torch.rand(n, generator=g) < 0.5] = -0.0
        x[torch.rand(n, generator=g) < 0.01] = 1.0
        return x
    if kind == "clustered":
        x = torch.randn(n, generator=g)
        x[n // 3: n // 3 + 3000] += 10.0   # every winner in a few tiles
        return x
    if kind == "relu_like":
        x = torch.relu(torch.randn(n, generator=g)) * torch.rand(n, generator=g)
        return x
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "ties", "equal", "ramp", "ramp_down", "zeros_signed",
                                  "clustered", "relu_like"])
@pytest.mark.parametrize("n,K", [(131072, 2048), (5000, 256), (100, 256), (2049, 2048),
                                 (40000, 1000)])
def test_topk_bit_exact(dsa, kind, n, K):
    say(f"topk {kind} n={n} K={K}")
    x = _topk_case(kind, n, seed=n + K)
    ctx = torch.tensor([n], dtype=torch.int32)
    got = dsa.dsa_topk(x[None].to(DEV).contiguous(), K, ctx.to(DEV), max_ctx=n)
    torch.cuda.synchronize()
    want = oracle.topk(x[None].numpy().astype(np.float32), K, ctx.numpy())
    assert np.array_equal(got.cpu().numpy(), want)


def test_topk_batched_ragged_rows(dsa):
    say("topk ragged multi-query rows")
    lens, nq = [9000, 300, 50000], [5, 300, 40]
    T = sum(nq)
    g = torch.Generator().manual_seed(3)
    s = torch.round(torch.randn(T, max(lens), generator=g) * 8) / 8
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(nq)]), dtype=torch.int32)
    ctx = torch.tensor(lens, dtype=torch.int32)
    got = dsa.dsa_topk(s.to(DEV), 2048, ctx.to(DEV), cu_q=cu_q.to(DEV), max_ctx=max(lens))
    torch.cuda.synchronize()
    want = oracle.topk(s.numpy(), 2048, ctx.numpy(), cu_q=cu_q.numpy())
    assert np.array_equal(got.cpu().numpy(), want)


def test_topk_one_million_rows(dsa):
    say("topk 4 rows x 1M")
    n, K = 1 << 20, 2048
    g = torch.Generator().manual_seed(4)
    s = torch.relu(torch.randn(4, n, generator=g)) * 3
    s[1] = torch.round(s[1] * 2) / 2            # heavy ties
    ctx = torch.full((4,), n, dtype=torch.int32)
    got = dsa.dsa_topk(s.to(DEV), K, ctx.to(DEV), max_ctx=n)
    torch.cuda.synchronize()
    want = oracle.topk(s.numpy(), K, ctx.numpy())
    assert np.array_equal(got.cpu().numpy(), want)


# Row lengths around each boundary of the selection paths, in one ragged
# batch whose longest row sets the report tile: direct rows (at most 16384
# positions), 32-position sub-tiles just above, sub-tiles smaller than the
# tile (with up to 1024 of them per row), and the longest row itself.
RAGGED_TOPK_LENS = [5000, 16384, 16385, 20000, 31000, 70000, 131071, 131072, 300000, 1 << 20]


def _with_counters(dsa, fn):
    cnt = torch.zeros(6, dtype=torch.int32, device=DEV)
    dsa.dsa_set_topk_counters(cnt)
    try:
        res = fn()
    finally:
        dsa.dsa_set_topk_counters(None)
    torch.cuda.synchronize()
    return res, cnt.cpu().numpy()


@pytest.mark.parametrize("kind", ["normal", "relu_like", "ties"])
def test_topk_ragged_rows_subtile_reports(dsa, kind):
    say(f"topk ragged rows {kind}: direct / sub-tile / full-tile paths")
    lens, K = RAGGED_TOPK_LENS, 2048
    L = max(lens)
    s = torch.stack([_topk_case(kind, L, seed=100 + i) for i in range(len(lens))])
    ctx = torch.tensor(lens, dtype=torch.int32)
    got, c = _with_counters(dsa, lambda: dsa.dsa_topk(s.to(DEV), K, ctx.to(DEV), max_ctx=L))
    want = oracle.topk(s.numpy(), K, ctx.numpy())
    assert np.array_equal(got.cpu().numpy(), want)
    n_direct = sum(1 for n in lens if K < n <= 16384)
    assert c[2] == n_direct
    assert c[0] + c[1] == len(lens) - n_direct
    if kind != "ties":   # continuous scores: every long row certifies
        assert c[1] == 0


def test_topk_clustered_rows_take_the_exact_fallback(dsa):
    """Every winner inside 3000 consecutive positions: the report unions
    fail their certification and the keys at or above each union's K-th
    best overflow the second chance's 4096 slots, so the rows take the
    exact select over the whole row."""
    say("topk clustered winners: exact fallback")
    lens, K = [40000, 131072, 70001], 2048
    L = max(lens)
    s = torch.zeros(len(lens), L)
    for i, n in enumerate(lens):
        s[i, :n] = _topk_case("clustered", n, seed=7 + i)   # winners packed in a few tiles
    ctx = torch.tensor(lens, dtype=torch.int32)
    got, c = _with_counters(dsa, lambda: dsa.dsa_topk(s.to(DEV), K, ctx.to(DEV), max_ctx=L))
    want = oracle.topk(s.numpy(), K, ctx.numpy())
    assert np.array_equal(got.cpu().numpy(), want)
    assert c[1] == len(lens) and c[5] == 0


@pytest.mark.parametrize("width", [300, 700, 1500])
def test_topk_failed_certification_takes_one_collection_sweep(dsa, width):
    """A few hundred winners packed together: the sub-tiles holding them
    report only 16 each, so the union fails its certification; the keys of
    each row at or above the union's K-th best (the packed winners plus
    about K others) fit 4096 slots and are selected in one collection sweep.
    Bit-exact against the oracle; every row takes that path."""
    say(f"topk failed certification, {width} packed winners: one collection sweep")
    lens, K = [40000, 131072, 70001, 300000], 2048
    L = max(lens)
    s = torch.zeros(len(lens), L)
    for i, n in enumerate(lens):
        g = torch.Generator().manual_seed(90 + i)
        x = torch.randn(n, generator=g)
        x[n // 2: n // 2 + width] += 10.0
        s[i, :n] = x
    ctx = torch.tensor(lens, dtype=torch.int32)
    got, c = _with_counters(dsa, lambda: dsa.dsa_topk(s.to(DEV), K, ctx.to(DEV), max_ctx=L))
    want = oracle.topk(s.numpy(), K, ctx.numpy())
    assert np.array_equal(got.cpu().numpy(), want)
    assert c[5] == len(lens) and c[1] == 0 and c[0] == 0, c


@pytest.mark.parametrize("kind", ["normal", "ties", "relu_like", "clustered", "equal"])
def test_topk_many_rows_take_the_row_sweeps(dsa, kind):
    """1024 rows and more (a prefill chunk) are selected by histogram and
    collection sweeps over each row; a key shared by more positions than the
    candidate buffer holds sends the row to the exact sweep select."""
    say(f"topk many rows {kind}")
    lens, nq, K = [30000, 1500, 9000], [700, 300, 100], 2048
    T, L = sum(nq), max(lens)
    s = torch.zeros(T, L)
    t = 0
    for b, (n_ctx, q) in enumerate(zip(lens, nq)):
        for i in range(q):
            p = n_ctx - q + i
            s[t, :p + 1] = _topk_case(kind, p + 1, seed=1000 * b + i)
            t += 1
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(nq)]), dtype=torch.int32)
    ctx = torch.tensor(lens, dtype=torch.int32)
    got, c = _with_counters(dsa, lambda: dsa.dsa_topk(s.to(DEV), K, ctx.to(DEV),
                                                      cu_q=cu_q.to(DEV), max_ctx=L))
    want = oracle.topk(s.numpy(), K, ctx.numpy(), cu_q=cu_q.numpy())
    assert np.array_equal(got.cpu().numpy(), want)
    n_sel = sum(1 for n_ctx, q in zip(lens, nq) for i in range(q) if n_ctx - q + i + 1 > K)
    n_long = sum(1 for n_ctx, q in zip(lens, nq) for i in range(q) if n_ctx - q + i + 1 >= 16384)
    assert c[0] == 0 and c[2] == 0 and c[1] + c[3] == n_sel and c[4] <= c[3]
    if kind == "equal":
        assert c[1] == n_sel
    elif kind in ("normal", "relu_like"):
        # long rows: one collection sweep from a sampled threshold
        assert c[3] == n_sel and c[4] == n_long


# --------------------------------------------------------------------------
# Gated sparse attention
# --------------------------------------------------------------------------

def _rand_idx(lens, nq, K, seed, full=False):
    g = np.random.default_rng(seed)
    rows = []
    for L, n in zip(lens, nq):
        for i in range(n):
            p = L - n + i
            keff = min(K, p + 1)
            sel = np.arange(p + 1) if full else np.sort(g.choice(p + 1, keff, replace=False))
            sel = sel[:keff]
            rows.append(np.concatenate([sel, -np.ones(K - keff, np.int64)]))
    return torch.tensor(np.array(rows), dtype=torch.int32)


@pytest.mark.parametrize("Hq,D,K,lens,nq,gated", [
    (8, 64, 256, [4096], [1], True),
    (64, 128, 2048, [131072], [1], True),
    (64, 128, 2048, [5000, 1500, 90000], [1, 1, 1], True),
    (64, 128, 2048, [1000], [1], True),          # K > context: padded
    (64, 128, 300, [4000], [64], False),         # multi-query rows, ungated
    (8, 64, 256, [700, 3000], [9, 17], True),
    # 40 queries of K = 4096: whole index rows per workgroup, capped at the
    # 2048 rows a workgroup stages, so two splits and the combine
    (64, 128, 4096, [6000], [40], True),
    (8, 64, 4096, [6000], [40], False),
])
def test_sparse_attn_indexed(dsa, Hq, D, K, lens, nq, gated):
    say(f"sparse_attn Hq={Hq} D={D} K={K} lens={lens} nq={nq}")
    w = wl("t", lens, nq, 4, 64, Hq, D, K, seed=21)
    inp = W.make_inputs(w)
    if not gated:
        inp["gate"] = None
    idx = _rand_idx(lens, nq, K, seed=5)
    d = to_dev(inp)
    cu_q = None if all(n == 1 for n in nq) else d["cu_q"]
    lse = torch.empty(w.T, Hq, device=DEV)
    out = dsa.dsa_sparse_attn(d["q"], d["k_cache"], d["v_cache"], idx.to(DEV), d["ctx_len"],
                              d["cu_ctx"], gate=d["gate"], cu_q=cu_q, max_ctx=max(lens), lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.sparse_attn(inp["q"], inp["k_cache"], inp["v_cache"], idx=idx,
                                      gate=inp["gate"], ctx_len=inp["ctx_len"], cu_q=inp["cu_q"],
                                      cu_ctx=inp["cu_ctx"])
    check_out(out, ref, ATOL_BF16)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)


def test_sparse_attn_skips_entries_outside_the_visible_range(dsa):
    """Index entries outside [0, p] (other negatives, positions past the
    query, the int32 maximum) are skipped like the -1 padding: the output
    equals the oracle's over the same rows with those entries set to -1, and
    no gather leaves the sequence."""
    say("sparse_attn out-of-range entries")
    lens, nq, K = [3000, 5000], [3, 2], 256
    w = wl("t", lens, nq, 4, 64, 64, 128, K, seed=23)
    inp = W.make_inputs(w)
    idx = _rand_idx(lens, nq, K, seed=6)
    bad = idx.clone()
    g = np.random.default_rng(7)
    t = 0
    for L, n in zip(lens, nq):
        for i in range(n):
            p = L - n + i
            cols = g.choice(K, 40, replace=False)
            vals = [p + 1, p + 1000, 2**31 - 1, -2, -100000, L, 10**9]
            for c, v in zip(cols, vals * 6):
                bad[t, c] = v
            t += 1
    clean = bad.clone()
    clean[(bad < 0) | (bad > torch.tensor(positions(lens, nq))[:, None])] = -1
    d = to_dev(inp)
    out = dsa.dsa_sparse_attn(d["q"], d["k_cache"], d["v_cache"], bad.to(DEV), d["ctx_len"],
                              d["cu_ctx"], gate=d["gate"], cu_q=d["cu_q"], max_ctx=max(lens))
    torch.cuda.synchronize()
    ref, _ = oracle.sparse_attn(inp["q"], inp["k_cache"], inp["v_cache"], idx=clean,
                                gate=inp["gate"], ctx_len=inp["ctx_len"], cu_q=inp["cu_q"],
                                cu_ctx=inp["cu_ctx"])
    check_out(out, ref, ATOL_BF16)


@pytest.mark.parametrize("lens,window", [([4096, 100, 129], 128), ([50000], 128), ([3], 128)])
def test_sparse_attn_window(dsa, lens, window):
    say(f"sparse_attn window={window} lens={lens}")
    w = wl("t", lens, [1] * len(lens), 4, 64, 64, 128, 0, seed=22)
    inp = W.make_inputs(w)
    d = to_dev(inp)
    out = dsa.dsa_sparse_attn(d["q"], d["k_cache"], d["v_cache"], None, d["ctx_len"], d["cu_ctx"],
                              window=window, max_ctx=max(lens))
    torch.cuda.synchronize()
    ref, _ = oracle.sparse_attn(inp["q"], inp["k_cache"], inp["v_cache"], window=window,
                                ctx_len=inp["ctx_len"], cu_ctx=inp["cu_ctx"])
    check_out(out, ref, ATOL_BF16)


def test_sparse_attn_window_many_queries(dsa):
    """100 query rows with a 3000-position window: each workgroup takes a
    whole window (more rows than the index staging holds, which window mode
    does not use), gated output, no split merge."""
    say("sparse_attn window=3000, 100 queries of one sequence")
    lens, nq = [6000], [100]
    w = wl("t", lens, nq, 4, 64, 64, 128, 0, seed=23)
    inp = W.make_inputs(w)
    d = to_dev(inp)
    lse = torch.empty(w.T, 64, device=DEV)
    out = dsa.dsa_sparse_attn(d["q"], d["k_cache"], d["v_cache"], None, d["ctx_len"], d["cu_ctx"],
                              gate=d["gate"], window=3000, cu_q=d["cu_q"], max_ctx=max(lens),
                              lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.sparse_attn(inp["q"], inp["k_cache"], inp["v_cache"], window=3000,
                                      gate=inp["gate"], ctx_len=inp["ctx_len"], cu_q=inp["cu_q"],
                                      cu_ctx=inp["cu_ctx"])
    check_out(out, ref, ATOL_BF16)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)


def _swa_layers(B, ntot, n, seed, device="cpu", Hq=64, D=128):
    return [{"q": W.randn_bf16((B, Hq, D), seed, f"swa{i}_q", device),
             "k": W.randn_bf16((ntot, D), seed, f"swa{i}_k", device),
             "v": W.randn_bf16((ntot, D), seed, f"swa{i}_v", device)} for i in range(n)]


@pytest.mark.parametrize("lens,gated", [([130, 5000, 777, 3, 128, 129, 64000, 4096], False),
                                        ([4096, 100], True)])
def test_swa_decode_layers_one_launch(dsa, lens, gated):
    """All sliding-window layers of a decode step in one launch, each layer
    with its own tensors, checked layer by layer against the oracle's window
    attention (contexts shorter than, equal to and longer than the window)."""
    say(f"swa_decode_layers: 5 layers, window 128, lens={lens}, gated={gated}")
    w = wl("t", lens, [1] * len(lens), 16, 128, 64, 128, 256, seed=42)
    inp = W.make_inputs(w)
    d = to_dev(inp)
    layers = _swa_layers(w.B, sum(lens), 5, 42)
    gates = None
    if gated:   # elementwise gates on some layers, per-head ones on none (one stride per call)
        gates = [W.randn_bf16((w.B, 64, 128), 42, f"swa{i}_g") if i % 2 == 0 else None
                 for i in range(5)]
    outs = dsa.dsa_swa_decode_layers([x["q"].to(DEV) for x in layers],
                                     [x["k"].to(DEV) for x in layers],
                                     [x["v"].to(DEV) for x in layers], d["ctx_len"], d["cu_ctx"],
                                     128, gates=None if gates is None else
                                     [None if g is None else g.to(DEV) for g in gates],
                                     max_ctx=max(lens))
    torch.cuda.synchronize()
    for i, x in enumerate(layers):
        ref, _ = oracle.sparse_attn(x["q"], x["k"], x["v"], window=128,
                                    gate=None if gates is None else gates[i],
                                    ctx_len=inp["ctx_len"], cu_ctx=inp["cu_ctx"])
        check_out(outs[i], ref, ATOL_BF16)


def test_hybrid_step_swa_layers_then_dsa_layer(dsa):
    """One decode step of the 5:1 hybrid at a small ragged shape, as the bench
    issues it: the five sliding-window layers (own K/V caches, ungated) in one
    launch through the prepared call, re-issued once, then the Gated DSA
    layer; every layer against the oracle."""
    say("hybrid step: 5 SWA layers (window 128) in one launch + 1 DSA layer, ragged batch")
    lens = [130, 5000, 777, 20000, 4096, 3, 129, 70000]
    w = wl("t", lens, [1] * len(lens), 16, 128, 64, 128, 2048, seed=41)
    inp = W.make_inputs(w)
    d = to_dev(inp)
    layers = _swa_layers(w.B, sum(lens), 5, 41)
    dl = [{k: v.to(DEV) for k, v in x.items()} for x in layers]
    outs = [torch.empty(w.B, 64, 128, dtype=torch.bfloat16, device=DEV) for _ in range(5)]
    call = dsa.prepare_swa_decode_layers([x["q"] for x in dl], [x["k"] for x in dl],
                                         [x["v"] for x in dl], d["ctx_len"], d["cu_ctx"],
                                         max(lens), outs, 128)
    call()
    call()  # re-issued: same result
    torch.cuda.synchronize()
    for i, x in enumerate(layers):
        ref, _ = oracle.sparse_attn(x["q"], x["k"], x["v"], window=128, ctx_len=inp["ctx_len"],
                                    cu_ctx=inp["cu_ctx"])
        check_out(outs[i], ref, ATOL_BF16)
    _layer_decode_check(dsa, w, inp, d)


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def _gate_for_oracle(gate, D):
    """The oracle takes an elementwise gate: a per-head gate [T, Hq] is
    expanded to [T, Hq, D] (each head's value on all its dims)."""
    if gate is None or gate.dim() == 3:
        return gate
    return gate[:, :, None].expand(-1, -1, D).contiguous()


def _check_topk_on_gpu_scores(idx_row, s_gpu_row, p, K):
    """Mode T: the layer's selection equals the oracle's selection on the
    very fp32 scores the layer computed (read back from its workspace)."""
    want = oracle.topk(np.ascontiguousarray(s_gpu_row[None, :p + 1], dtype=np.float32), K,
                       np.array([p + 1], np.int32))[0]
    assert np.array_equal(idx_row, want), "selection differs from the Top-K of the GPU's scores"


def _layer_decode_check(dsa, w, inp_cpu, d, seqs=None, atol=ATOL_BF16, gate=None):
    B = w.B
    L = max(w.ctx_lens)
    gate_dev = d["gate"] if gate is None else gate.to(DEV)
    gate_cpu = _gate_for_oracle(inp_cpu["gate"] if gate is None else gate, w.D)
    idx = torch.empty(B, w.K, dtype=torch.int32, device=DEV)
    ws = torch.empty(dsa.dsa_layer_decode_workspace_size(B, L, w.K, w.Hq, w.D), dtype=torch.uint8,
                     device=DEV)
    out = dsa.dsa_layer_decode(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["q"], d["k_cache"],
                               d["v_cache"], gate_dev, w.K, d["ctx_len"], d["cu_ctx"],
                               max_ctx=L, idx_out=idx, ws=ws)
    torch.cuda.synchronize()
    idx_c = idx.cpu().numpy()
    seqs = range(B) if seqs is None else seqs
    rows = torch.tensor(list(seqs), dtype=torch.int64, device=DEV)
    s_gpu = dsa.layer_scores(ws, B, L)[rows].cpu().numpy()
    ndiff = 0
    for i, b in enumerate(seqs):
        Lb = w.ctx_lens[b]
        r0 = int(sum(w.ctx_lens[:b]))
        ks = None if inp_cpu["k_scale"] is None else inp_cpu["k_scale"][r0:r0 + Lb]
        s_ref = oracle.index_scores(inp_cpu["q_idx"][b:b + 1], inp_cpu["w"][b:b + 1],
                                    inp_cpu["k_idx"][r0:r0 + Lb], ks,
                                    ctx_len=np.array([Lb], np.int32))[0]
        sel = check_index_row(idx_c[b], Lb - 1, w.K)
        _check_topk_on_gpu_scores(idx_c[b], s_gpu[i], Lb - 1, w.K)
        ndiff += check_set_band(sel, s_ref, Lb - 1, w.K)
        g = None if gate_cpu is None else gate_cpu[b:b + 1]
        ref, _ = oracle.sparse_attn(inp_cpu["q"][b:b + 1], inp_cpu["k_cache"][r0:r0 + Lb],
                                    inp_cpu["v_cache"][r0:r0 + Lb], idx=idx_c[b:b + 1],
                                    gate=g, ctx_len=np.array([Lb], np.int32))
        check_out(out[b:b + 1], ref, atol)
    return ndiff


def test_layer_decode_tiny(dsa):
    say("layer_decode tiny ctx 4096")
    w = W.tiny_decode()
    inp = W.make_inputs(w)
    _layer_decode_check(dsa, w, inp, to_dev(inp))


def test_layer_decode_ragged_batch_and_short_rows(dsa):
    say("layer_decode ragged batch with rows shorter than K")
    w = wl("t", [3000, 100, 70000, 2048, 2049], [1] * 5, 16, 128, 64, 128, 2048, seed=31,
           plant_frac=0.05)
    inp = W.make_inputs(w)
    _layer_decode_check(dsa, w, inp, to_dev(inp))


def test_layer_decode_ragged_lengths_take_the_fast_paths(dsa):
    say("layer_decode ragged lengths 4096..400000: direct and sub-tile selection")
    lens = [4096, 9000, 17000, 24000, 60000, 150000, 400000]
    w = wl("t", lens, [1] * len(lens), 16, 128, 64, 128, 2048, seed=51, plant_frac=0.05)
    inp = W.make_inputs(w)
    _, c = _with_counters(dsa, lambda: _layer_decode_check(dsa, w, inp, to_dev(inp)))
    assert c[2] == 2 and c[0] == len(lens) - 2 and c[1] == 0


def test_layer_decode_clustered_winners_take_the_fallbacks(dsa):
    """Winners packed into a few hundred consecutive positions break the
    per-sub-tile certification; in the decode layer of few sequences the
    selection runs inside every split workgroup of the attention launch, so
    both second chances run there: a cluster of 1500 positions (its failing
    sub-tiles leave at most 3152 keys at or above the union's threshold)
    takes the one collection sweep, a cluster of 3500 (4688 > 4096) the
    exact select over the row.  Index rows stay bit-exact against the
    oracle's Top-K of the layer's own scores, outputs within tolerance."""
    say("layer_decode clustered winners: collection sweep and exact select in the fused launch")
    lens = [40000, 60000]
    w = wl("t", lens, [1, 1], 16, 128, 64, 128, 2048, seed=61)
    inp = W.make_inputs(w)
    k = inp["k_idx"].float()
    k[5000:6500] *= 8.0                    # sequence 0
    k[lens[0] + 10000:lens[0] + 13500] *= 8.0  # sequence 1
    inp["k_idx"] = k.to(torch.bfloat16)    # powers of two: exact
    _, c = _with_counters(dsa, lambda: _layer_decode_check(dsa, w, inp, to_dev(inp)))
    assert c[5] == 1 and c[1] == 1 and c[0] == 0, c


def test_layer_decode_selection_widths_in_the_fused_launch(dsa):
    """In the decode layer of few sequences a union of at most 8192 report
    candidates is selected by the first 8 waves of each split workgroup (16
    slots per thread) and a larger one by all 16: a row of 131072 positions
    (512 sub-tiles of 256) next to a row of 100000 (782 sub-tiles of 128,
    in the wider layout) in one launch, then the same two rows with their
    winners clustered so that the first takes the collection sweep and the
    second the exact select, both run by the whole block.  Index rows stay
    bit-exact against the oracle's Top-K of the layer's own scores."""
    say("layer_decode selection widths: 8-wave and 16-wave unions, fallbacks after the 8-wave one")
    lens = [131072, 100000]
    w = wl("t", lens, [1, 1], 16, 128, 64, 128, 2048, seed=67, plant_frac=0.05)
    inp = W.make_inputs(w)
    _, c = _with_counters(dsa, lambda: _layer_decode_check(dsa, w, inp, to_dev(inp)))
    assert c[0] == 2 and c[1] == 0 and c[5] == 0, c
    w = wl("t", lens, [1, 1], 16, 128, 64, 128, 2048, seed=68)
    inp = W.make_inputs(w)
    k = inp["k_idx"].float()
    k[20000:21500] *= 8.0                      # sequence 0: collection sweep
    k[lens[0] + 30000:lens[0] + 33500] *= 8.0  # sequence 1: exact select
    inp["k_idx"] = k.to(torch.bfloat16)        # powers of two: exact
    _, c = _with_counters(dsa, lambda: _layer_decode_check(dsa, w, inp, to_dev(inp)))
    assert c[5] == 1 and c[1] == 1 and c[0] == 0, c


def test_layer_decode_2m_context_full_union(dsa):
    """One sequence of 2^21 positions (fp8 keys): 1024 sub-tiles of 2048,
    16384 report candidates, selected by all 16 waves of each split
    workgroup inside the attention's launch."""
    say("layer_decode 2M context fp8: 16384-candidate union in the fused launch")
    w = wl("t", [1 << 21], [1], 32, 128, 64, 128, 2048, key_dtype="fp8", seed=69)
    inp = W.make_inputs(w)
    _, c = _with_counters(dsa, lambda: _layer_decode_check(dsa, w, inp, to_dev(inp)))
    assert c[0] == 1 and c[1] == 0 and c[5] == 0, c


def test_layer_decode_large_batch_takes_the_row_sweeps(dsa):
    """1024 sequences and more: the indexer writes plain scores and every row
    is selected by sweeps over them (no candidate reports)."""
    say("layer_decode batch of 1024 ragged rows: row-sweep selection")
    g = np.random.default_rng(77)
    lens = [int(x) for x in g.integers(300, 3000, size=1024)]
    w = wl("t", lens, [1] * len(lens), 4, 64, 8, 64, 256, seed=52)
    inp = W.make_inputs(w)
    sample = sorted(g.choice(len(lens), size=48, replace=False).tolist())
    _, c = _with_counters(dsa, lambda: _layer_decode_check(dsa, w, inp, to_dev(inp),
                                                           seqs=sample))
    assert c[3] == len(lens) and c[0] == 0 and c[2] == 0 and c[1] == 0


def test_layer_decode_k_at_least_context_is_dense_attention(dsa):
    say("layer_decode K >= ctx equals gated dense attention")
    w = wl("t", [1500], [1], 32, 128, 64, 128, 2048, seed=32)
    inp = W.make_inputs(w)
    d = to_dev(inp)
    idx = torch.empty(1, 2048, dtype=torch.int32, device=DEV)
    out = dsa.dsa_layer_decode(d["q_idx"], d["w"], d["k_idx"], None, d["q"], d["k_cache"],
                               d["v_cache"], d["gate"], 2048, d["ctx_len"], d["cu_ctx"],
                               max_ctx=1500, idx_out=idx)
    torch.cuda.synchronize()
    assert idx.cpu()[0, :1500].tolist() == list(range(1500))
    assert bool((idx.cpu()[0, 1500:] == -1).all())
    qd = inp["q"].double().permute(1, 0, 2)[None]
    kd = inp["k_cache"].double()[None, None].expand(1, 64, 1500, 128)
    vd = inp["v_cache"].double()[None, None].expand(1, 64, 1500, 128)
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd)[0].permute(1, 0, 2)
    ref = ref * torch.sigmoid(inp["gate"].double())
    check_out(out, ref.numpy(), ATOL_BF16)


def test_layer_decode_128k_full_size(dsa):
    say("layer_decode 128K context, 32x128 indexer, planted keys (bench workload)")
    w = W.decode_128k()
    inp = W.make_inputs(w)
    nd = _layer_decode_check(dsa, w, inp, to_dev(inp))
    say(f"  positions differing within the band: {nd}")


def test_layer_decode_deterministic(dsa):
    """100 reruns of the 128K decode layer, the workspace alternately zeroed
    and poisoned with 0xFF before each: every output and index row equal to
    the first bit for bit (races in LDS or atomics, or reads of unwritten
    scratch, would show as differences)."""
    say("layer_decode determinism: 100 reruns, poisoned / zeroed workspace")
    w = W.decode_128k()
    inp = W.make_inputs(w)
    d = to_dev(inp)
    L = w.ctx_lens[0]
    ws = torch.empty(dsa.dsa_layer_decode_workspace_size(1, L, w.K, w.Hq, w.D),
                     dtype=torch.uint8, device=DEV)
    n = 100
    outs = torch.empty(n, 1, w.Hq, w.D, dtype=torch.bfloat16, device=DEV)
    idxs = torch.empty(n, 1, w.K, dtype=torch.int32, device=DEV)
    for r in range(n):
        ws.fill_(255 if r % 2 else 0)
        dsa.dsa_layer_decode(d["q_idx"], d["w"], d["k_idx"], None, d["q"], d["k_cache"],
                             d["v_cache"], d["gate"], w.K, d["ctx_len"], d["cu_ctx"],
                             max_ctx=L, out=outs[r], idx_out=idxs[r], ws=ws)
    torch.cuda.synchronize()
    o16 = outs.view(torch.int16)
    assert torch.equal(o16, o16[:1].expand_as(o16))
    assert torch.equal(idxs, idxs[:1].expand_as(idxs))


def test_layer_decode_1m_fp8_batched_sampled(dsa):
    say("layer_decode 32 x 1M fp8 keys (sampled sequences 0 and 31)")
    w = W.decode_1m_b32_fp8()
    inp_dev = W.make_inputs(w, device=DEV)
    L = w.ctx_lens[0]
    # the oracle reads the sampled sequences' slices of the same generated tensors
    inp = {}
    for k, v in inp_dev.items():
        inp[k] = None if v is None else v.detach()
    samp = [0, 31]
    cpu_inp = {
        "q_idx": cpu(inp["q_idx"]), "w": cpu(inp["w"]), "q": cpu(inp["q"]),
        "gate": cpu(inp["gate"]),
        "k_idx": None, "k_scale": None, "k_cache": None, "v_cache": None,
    }
    idx = torch.empty(w.B, w.K, dtype=torch.int32, device=DEV)
    ws = torch.empty(dsa.dsa_layer_decode_workspace_size(w.B, L, w.K, w.Hq, w.D),
                     dtype=torch.uint8, device=DEV)
    out = dsa.dsa_layer_decode(inp["q_idx"], inp["w"], inp["k_idx"], inp["k_scale"], inp["q"],
                               inp["k_cache"], inp["v_cache"], inp["gate"], w.K, inp["ctx_len"],
                               inp["cu_ctx"], max_ctx=L, idx_out=idx, ws=ws)
    torch.cuda.synchronize()
    idx_c = idx.cpu().numpy()
    s_gpu = dsa.layer_scores(ws, w.B, L)
    for b in samp:
        _check_topk_on_gpu_scores(idx_c[b], s_gpu[b].cpu().numpy(), L - 1, w.K)
        r0 = b * L
        s_ref = oracle.index_scores(cpu_inp["q_idx"][b:b + 1], cpu_inp["w"][b:b + 1],
                                    cpu(inp["k_idx"][r0:r0 + L]), cpu(inp["k_scale"][r0:r0 + L]),
                                    ctx_len=np.array([L], np.int32))[0]
        sel = check_index_row(idx_c[b], L - 1, w.K)
        check_set_band(sel, s_ref, L - 1, w.K)
        rows = torch.from_numpy(sel.astype(np.int64)) + r0
        kc = cpu(inp["k_cache"][rows.to(DEV)])
        vc = cpu(inp["v_cache"][rows.to(DEV)])
        ref, _ = oracle.sparse_attn(cpu_inp["q"][b:b + 1], kc, vc,
                                    idx=np.arange(len(sel), dtype=np.int32)[None],
                                    gate=cpu_inp["gate"][b:b + 1],
                                    ctx_len=np.array([len(sel)], np.int32))
        check_out(out[b:b + 1], ref, ATOL_FP8)


def _layer_prefill_check(dsa, w, inp, d, rows=None, ws_bytes=None, gate=None):
    """One prefill call, then per sampled row: the selection against the Top-K
    of the GPU's own fp32 scores (bit-exact; one-pass calls only), against
    the oracle's scores within the near-tie band, and the attention output
    against the oracle on the GPU's selection.  Returns (out, idx)."""
    L = max(w.ctx_lens)
    gate_dev = d["gate"] if gate is None else gate.to(DEV)
    gate_cpu = _gate_for_oracle(cpu(inp["gate"]) if gate is None else gate, w.D)
    full = dsa.dsa_layer_prefill_workspace_size(w.B, w.T, L, w.K, w.Hq, w.D)
    ws = torch.empty(full if ws_bytes is None else ws_bytes, dtype=torch.uint8, device=DEV)
    idx = torch.empty(w.T, w.K, dtype=torch.int32, device=DEV)
    out = dsa.dsa_layer_prefill(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["q"],
                                d["k_cache"], d["v_cache"], gate_dev, w.K, d["cu_q"],
                                d["ctx_len"], d["cu_ctx"], max_q=max(w.n_q), max_ctx=L,
                                idx_out=idx, ws=ws, q_scale=d.get("q_scale"))
    torch.cuda.synchronize()
    idx_c = idx.cpu().numpy()
    pos = positions(w.ctx_lens, w.n_q)
    seq_of = np.repeat(np.arange(w.B), w.n_q)
    rows = list(range(w.T)) if rows is None else list(rows)
    cu_ctx = np.concatenate([[0], np.cumsum(w.ctx_lens)])
    one_pass = ws.numel() >= full
    if one_pass:
        sel_rows = torch.tensor(rows, dtype=torch.int64, device=DEV)
        s_gpu = dsa.layer_scores(ws, w.T, L)[sel_rows].cpu().numpy()
    k_idx = cpu(inp["k_idx"])       # one host copy of the key cache, sliced per row
    k_scale = cpu(inp["k_scale"])
    for i, t in enumerate(rows):
        b, p = int(seq_of[t]), pos[t]
        r0 = int(cu_ctx[b])
        ks = None if k_scale is None else k_scale[r0:r0 + p + 1]
        # the pinned indexer score on a one-query descriptor: the query at p sees 0..p
        qs = inp.get("q_scale")
        s_ref = oracle.index_scores(cpu(inp["q_idx"][t:t + 1]), cpu(inp["w"][t:t + 1]),
                                    k_idx[r0:r0 + p + 1], ks,
                                    ctx_len=np.array([p + 1], np.int32),
                                    q_scale=None if qs is None else cpu(qs[t:t + 1]))[0]
        sel = check_index_row(idx_c[t], p, w.K)
        if one_pass:
            _check_topk_on_gpu_scores(idx_c[t], s_gpu[i], p, w.K)
        check_set_band(sel, s_ref, p, w.K)
        rr = torch.from_numpy(sel.astype(np.int64)) + r0
        dev = inp["k_cache"].device
        g = None if gate_cpu is None else gate_cpu[t:t + 1]
        ref, _ = oracle.sparse_attn(cpu(inp["q"][t:t + 1]), cpu(inp["k_cache"][rr.to(dev)]),
                                    cpu(inp["v_cache"][rr.to(dev)]),
                                    idx=np.arange(len(sel), dtype=np.int32)[None],
                                    gate=g, ctx_len=np.array([len(sel)], np.int32))
        check_out(out[t:t + 1], ref, ATOL_BF16 if inp["k_scale"] is None else ATOL_FP8)
    return out, idx


def test_layer_prefill_small(dsa):
    say("layer_prefill 2 sequences, short and long rows")
    w = wl("t", [6000, 2500], [300, 2500], 16, 128, 64, 128, 2048, seed=41)
    inp = W.make_inputs(w)
    _layer_prefill_check(dsa, w, inp, to_dev(inp), rows=list(range(0, w.T, 37)) + [w.T - 1])


@pytest.mark.parametrize("lens,nq,H_I,d_I", [([6000, 2500], [300, 2500], 16, 128),
                                             ([4096], [64], 4, 64)])
def test_layer_prefill_fp8_queries(dsa, lens, nq, H_I, d_I):
    """fp8 query heads and keys: the fp8 MFMA indexer inside the layer."""
    say(f"layer_prefill fp8 queries lens={lens} nq={nq} H_I={H_I}")
    w = wl("t", lens, nq, H_I, d_I, 64 if d_I == 128 else 8, d_I, 2048 if d_I == 128 else 256,
           key_dtype="fp8", q_dtype="fp8", seed=45)
    inp = W.make_inputs(w)
    rows = list(range(0, w.T, 29)) + [w.T - 1]
    _layer_prefill_check(dsa, w, inp, to_dev(inp), rows=rows)


def test_layer_prefill_fp8_queries_sub_chunks(dsa):
    """fp8 query heads through the sub-chunked prefill (pointer offsets of
    one-byte query rows and of their scales)."""
    say("layer_prefill fp8 queries in sub-chunks")
    w = wl("t", [5000, 1200], [700, 400], 16, 128, 64, 128, 2048, key_dtype="fp8",
           q_dtype="fp8", seed=46)
    inp = W.make_inputs(w)
    d = to_dev(inp)
    L = max(w.ctx_lens)
    small = (dsa.dsa_layer_prefill_workspace_size(w.B, 300, L, w.K, w.Hq, w.D) +
             dsa.dsa_layer_prefill_min_workspace_size(w.B, L, w.K, w.Hq, w.D))
    _layer_prefill_check(dsa, w, inp, d, rows=[0, 299, 300, 699, 700, 1099], ws_bytes=small)


def test_layer_prefill_tiny_shape(dsa):
    say("layer_prefill tiny shape (4x64 indexer, 8 heads x 64)")
    w = wl("t", [4096], [64], 4, 64, 8, 64, 256, seed=42)
    inp = W.make_inputs(w)
    _layer_prefill_check(dsa, w, inp, to_dev(inp))


@pytest.mark.parametrize("fp8", [False, True])
def test_layer_prefill_8k_chunk_sampled(dsa, fp8):
    say(f"layer_prefill 8192 queries on a 131072-token context (sampled rows), fp8={fp8}")
    w = W.prefill_8k_fp8() if fp8 else W.prefill_8k()
    inp = W.make_inputs(w, device=DEV)
    # 64 evenly spaced rows, the first and the last included: every compute
    # wave of the indexer's 28-query workgroups is sampled
    rows = np.unique(np.linspace(0, w.T - 1, 64).round().astype(int)).tolist()
    assert len(rows) == 64 and rows[0] == 0 and rows[-1] == w.T - 1
    assert len({(r % 28) // 4 for r in rows}) == 7
    _layer_prefill_check(dsa, w, inp, inp, rows=rows)


def test_layer_decode_replays_as_a_hip_graph(dsa):
    """The decode layer launches kernels only (no memset, no host sync), so it
    can be captured into a HIP graph.  Three replays, with eager layer calls
    on other buffers and host synchronisations between them, each equal the
    eager result bit for bit (the path is deterministic)."""
    say("layer_decode captured as a HIP graph, replayed 3x")
    w = wl("t", [40000, 23000], [1, 1], 32, 128, 64, 128, 2048, seed=51, plant_frac=0.05,
           plant_mult=4.0)
    inp = W.make_inputs(w, device=DEV)
    other = W.make_inputs(w, device=DEV, seed_offset=1)
    L = max(w.ctx_lens)
    cap = torch.cuda.Stream()

    def setup(d):
        ws = torch.empty(dsa.dsa_layer_decode_workspace_size(w.B, L, w.K, w.Hq, w.D),
                         dtype=torch.uint8, device=DEV)
        out = torch.empty_like(d["q"])
        idx = torch.empty(w.B, w.K, dtype=torch.int32, device=DEV)
        call = dsa.prepare_layer_decode(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["q"],
                                        d["k_cache"], d["v_cache"], d["gate"], w.K, d["ctx_len"],
                                        d["cu_ctx"], L, out, ws, idx_out=idx, stream=cap)
        return call, out, idx

    call, out, idx = setup(inp)
    call_o, out_o, idx_o = setup(other)
    call()
    torch.cuda.synchronize()
    want_out, want_idx = out.clone(), idx.clone()
    call_o()
    torch.cuda.synchronize()
    want_out_o = out_o.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        idx.fill_(-7)
        torch.cuda.synchronize()
        with torch.cuda.stream(cap):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_out), f"replay {rep}: output differs from eager"
        assert torch.equal(idx, want_idx), f"replay {rep}: indices differ from eager"
        out_o.zero_()
        call_o()  # eager work on other buffers between replays
        torch.cuda.synchronize()
        assert torch.equal(out_o, want_out_o)


# --------------------------------------------------------------------------
# Per-head scalar gate, poisoned workspaces, prefill sub-chunks, side streams
# --------------------------------------------------------------------------

@pytest.mark.parametrize("lens,nq,K", [([131072], [1], 2048),      # split + combine kernel
                                       ([6000], [40], 2048),       # one workgroup per row
                                       ([4096, 700], [1, 1], 256)])
def test_sparse_attn_per_head_gate(dsa, lens, nq, K):
    """gate_stride_d = 0: one gate value per head, applied to all its dims."""
    say(f"sparse_attn per-head gate lens={lens} nq={nq} K={K}")
    w = wl("t", lens, nq, 4, 64, 64, 128, K, seed=24)
    inp = W.make_inputs(w)
    gate = W.randn_bf16((w.T, 64), 24, "head_gate")
    idx = _rand_idx(lens, nq, K, seed=6)
    d = to_dev(inp)
    cu_q = None if all(n == 1 for n in nq) else d["cu_q"]
    out = dsa.dsa_sparse_attn(d["q"], d["k_cache"], d["v_cache"], idx.to(DEV), d["ctx_len"],
                              d["cu_ctx"], gate=gate.to(DEV), cu_q=cu_q, max_ctx=max(lens))
    torch.cuda.synchronize()
    ref, _ = oracle.sparse_attn(inp["q"], inp["k_cache"], inp["v_cache"], idx=idx,
                                gate=_gate_for_oracle(gate, 128), ctx_len=inp["ctx_len"],
                                cu_q=inp["cu_q"], cu_ctx=inp["cu_ctx"])
    check_out(out, ref, ATOL_BF16)


def test_layer_decode_per_head_gate(dsa):
    say("layer_decode with one gate value per head")
    w = wl("t", [40000, 3000], [1, 1], 32, 128, 64, 128, 2048, seed=33, plant_frac=0.05)
    inp = W.make_inputs(w)
    gate = W.randn_bf16((w.B, w.Hq), 33, "head_gate")
    _layer_decode_check(dsa, w, inp, to_dev(inp), gate=gate)


def test_layer_prefill_per_head_gate(dsa):
    say("layer_prefill with one gate value per head")
    w = wl("t", [5000], [150], 16, 128, 64, 128, 2048, seed=34)
    inp = W.make_inputs(w)
    gate = W.randn_bf16((w.T, w.Hq), 34, "head_gate")
    _layer_prefill_check(dsa, w, inp, to_dev(inp), rows=list(range(0, w.T, 13)) + [w.T - 1],
                         gate=gate)


# --------------------------------------------------------------------------
# Seeded random shapes: every supported indexer and attention shape, K,
# key dtype and gate kind, ragged batches mixing rows shorter than K,
# direct rows, sub-tile rows and lengths at the sub-tile-size boundaries
# --------------------------------------------------------------------------

_IDX_SHAPES = [(4, 64), (16, 128), (32, 128)]
_ATT_SHAPES = [(8, 64), (64, 128)]
_BOUNDARY_LENS = [16384, 16385, 32768, 65536, 65537, 131071, 131072]


def _random_case(seed, prefill):
    g = np.random.default_rng(seed)
    H_I, d_I = _IDX_SHAPES[g.integers(len(_IDX_SHAPES))]
    Hq, D = _ATT_SHAPES[g.integers(len(_ATT_SHAPES))]
    K = int(g.choice([16, 64, 256, 1000, 2048, 4096]))
    key = "fp8" if g.random() < 0.5 else "bf16"
    q8 = prefill and key == "fp8" and d_I == 128 and g.random() < 0.5
    B = int(g.integers(1, 5 if prefill else 7))
    lens, nq = [], []
    for _ in range(B):
        kind = int(g.integers(5))
        if kind == 0:
            n = int(g.integers(1, K + 1))
        elif kind == 1:
            n = int(g.integers(K + 1, 16385)) if K < 16384 else 16384
        elif kind == 2:
            n = int(g.integers(16385, 70000))
        elif kind == 3:
            n = int(g.integers(70000, 300000 if not prefill else 140000))
        else:
            n = int(g.choice(_BOUNDARY_LENS))
        lens.append(n)
        nq.append(int(g.integers(1, min(n, 40) + 1)) if prefill else 1)
    gate_kind = int(g.integers(2))   # 0: elementwise, 1: one value per head
    w = wl(f"rand{seed}", lens, nq, H_I, d_I, Hq, D, K, key_dtype=key,
           q_dtype="fp8" if q8 else "bf16", seed=seed,
           plant_frac=0.05 if g.random() < 0.5 else 0.0)
    return w, gate_kind


@pytest.mark.parametrize("seed", list(range(1000, 1012)))
def test_layer_decode_random_shapes(dsa, seed):
    w, gate_kind = _random_case(seed, prefill=False)
    say(f"layer_decode random seed={seed}: lens={w.ctx_lens} H_I={w.H_I} d_I={w.d_I} "
        f"Hq={w.Hq} D={w.D} K={w.K} keys={w.key_dtype} gate={'head' if gate_kind else 'elem'}")
    inp = W.make_inputs(w)
    gate = W.randn_bf16((w.B, w.Hq), seed, "head_gate") if gate_kind else None
    _layer_decode_check(dsa, w, inp, to_dev(inp), gate=gate,
                        atol=ATOL_FP8 if w.key_dtype == "fp8" else ATOL_BF16)


@pytest.mark.parametrize("seed", list(range(2000, 2006)))
def test_layer_prefill_random_shapes(dsa, seed):
    w, gate_kind = _random_case(seed, prefill=True)
    say(f"layer_prefill random seed={seed}: lens={w.ctx_lens} nq={w.n_q} H_I={w.H_I} "
        f"d_I={w.d_I} Hq={w.Hq} D={w.D} K={w.K} keys={w.key_dtype} queries={w.q_dtype} "
        f"gate={'head' if gate_kind else 'elem'}")
    inp = W.make_inputs(w)
    gate = W.randn_bf16((w.T, w.Hq), seed, "head_gate") if gate_kind else None
    rows = sorted(set(list(range(0, w.T, max(1, w.T // 12))) + [w.T - 1]))
    _layer_prefill_check(dsa, w, inp, to_dev(inp), rows=rows, gate=gate)


def _run_decode(dsa, w, d, ws):
    idx = torch.empty(w.B, w.K, dtype=torch.int32, device=DEV)
    out = dsa.dsa_layer_decode(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["q"], d["k_cache"],
                               d["v_cache"], d["gate"], w.K, d["ctx_len"], d["cu_ctx"],
                               max_ctx=max(w.ctx_lens), idx_out=idx, ws=ws)
    return out, idx


def test_layer_decode_poisoned_workspace(dsa):
    """A workspace filled with 0xFF bytes (NaN scores, -1 words) gives the
    same bits as a zeroed one: no step reads scratch it did not write."""
    say("layer_decode 128K: workspace poisoned with 0xFF vs zeroed")
    w = W.decode_128k()
    d = W.make_inputs(w, device=DEV)
    L = max(w.ctx_lens)
    nb = dsa.dsa_layer_decode_workspace_size(w.B, L, w.K, w.Hq, w.D)
    ws0 = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    ws1 = torch.full((nb,), 255, dtype=torch.uint8, device=DEV)
    o0, i0 = _run_decode(dsa, w, d, ws0)
    o1, i1 = _run_decode(dsa, w, d, ws1)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))


def _prefill_small():
    return wl("t", [6000, 2500, 900], [300, 2500, 150], 16, 128, 64, 128, 2048, seed=43)


def _run_prefill(dsa, w, d, ws):
    idx = torch.empty(w.T, w.K, dtype=torch.int32, device=DEV)
    out = dsa.dsa_layer_prefill(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["q"],
                                d["k_cache"], d["v_cache"], d["gate"], w.K, d["cu_q"],
                                d["ctx_len"], d["cu_ctx"], max_q=max(w.n_q),
                                max_ctx=max(w.ctx_lens), idx_out=idx, ws=ws)
    return out, idx


def test_layer_prefill_poisoned_workspace(dsa):
    say("layer_prefill: workspace poisoned with 0xFF vs zeroed")
    w = _prefill_small()
    d = W.make_inputs(w, device=DEV)
    nb = dsa.dsa_layer_prefill_workspace_size(w.B, w.T, max(w.ctx_lens), w.K, w.Hq, w.D)
    o0, i0 = _run_prefill(dsa, w, d, torch.zeros(nb, dtype=torch.uint8, device=DEV))
    o1, i1 = _run_prefill(dsa, w, d, torch.full((nb,), 255, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(i0, i1)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))


def test_layer_prefill_sub_chunks(dsa):
    """A workspace too small for the score array of all rows: the library runs
    the rows in sub-chunks (here at least three, crossing sequence
    boundaries).  Every step is row-wise and the chunks keep the Top-K and
    attention plans of the one-pass call at these sizes, so the result is
    bit-identical to it; sampled rows are also checked against the oracle.
    The chunked call runs on a poisoned (0xFF) workspace."""
    say("layer_prefill in sub-chunks (workspace for ~900 rows, 2950 rows)")
    w = _prefill_small()
    inp = W.make_inputs(w)
    d = to_dev(inp)
    L = max(w.ctx_lens)
    full = dsa.dsa_layer_prefill_workspace_size(w.B, w.T, L, w.K, w.Hq, w.D)
    small = (dsa.dsa_layer_prefill_workspace_size(w.B, 900, L, w.K, w.Hq, w.D) +
             dsa.dsa_layer_prefill_min_workspace_size(w.B, L, w.K, w.Hq, w.D))
    assert small < full / 3
    o_full, i_full = _run_prefill(dsa, w, d, torch.empty(full, dtype=torch.uint8, device=DEV))
    o_sub, i_sub = _run_prefill(dsa, w, d,
                                torch.full((small,), 255, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(i_full, i_sub)
    assert torch.equal(o_full.view(torch.int16), o_sub.view(torch.int16))
    rows = [0, 299, 300, 899, 900, 1799, 1800, 2799, 2800, 2949]
    _layer_prefill_check(dsa, w, inp, d, rows=rows, ws_bytes=small)


def test_layer_prefill_smallest_workspace(dsa):
    """The least accepted workspace: one query row per sub-chunk."""
    say("layer_prefill with the minimum workspace (one row per sub-chunk)")
    w = wl("t", [3000, 2100], [5, 4], 16, 128, 64, 128, 2048, seed=44)
    inp = W.make_inputs(w)
    d = to_dev(inp)
    L = max(w.ctx_lens)
    nb = dsa.dsa_layer_prefill_min_workspace_size(w.B, L, w.K, w.Hq, w.D)
    _layer_prefill_check(dsa, w, inp, d, ws_bytes=nb)
    with pytest.raises(dsa.DSAError):
        _run_prefill(dsa, w, d, torch.empty(nb - 256, dtype=torch.uint8, device=DEV))


def test_index_checks_report_nothing_on_clean_calls(dsa):
    """With the index-row checks on, a ragged decode layer, a sub-chunked
    prefill layer, a batched dsa_topk and an attention call over the decode
    layer's own rows report no violation, and every row is checked once."""
    say("index-row checks on clean decode, prefill, topk and attention calls")
    c = torch.zeros(4, dtype=torch.int32, device=DEV)
    dsa.dsa_set_index_checks(c)
    try:
        w = wl("t", [3000, 100, 70000, 2048, 2049], [1] * 5, 16, 128, 64, 128, 2048, seed=31,
               plant_frac=0.05)
        d = to_dev(W.make_inputs(w))
        L = max(w.ctx_lens)
        idx = torch.empty(w.B, w.K, dtype=torch.int32, device=DEV)
        ws = torch.empty(dsa.dsa_layer_decode_workspace_size(w.B, L, w.K, w.Hq, w.D),
                         dtype=torch.uint8, device=DEV)
        dsa.dsa_layer_decode(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["q"], d["k_cache"],
                             d["v_cache"], d["gate"], w.K, d["ctx_len"], d["cu_ctx"], max_ctx=L,
                             idx_out=idx, ws=ws)
        dsa.dsa_sparse_attn(d["q"], d["k_cache"], d["v_cache"], idx, d["ctx_len"], d["cu_ctx"],
                            gate=d["gate"], max_ctx=L)
        rows = 2 * w.B
        w2 = _prefill_small()
        d2 = W.make_inputs(w2, device=DEV)
        L2 = max(w2.ctx_lens)
        small = (dsa.dsa_layer_prefill_workspace_size(w2.B, 900, L2, w2.K, w2.Hq, w2.D) +
                 dsa.dsa_layer_prefill_min_workspace_size(w2.B, L2, w2.K, w2.Hq, w2.D))
        _run_prefill(dsa, w2, d2, torch.empty(small, dtype=torch.uint8, device=DEV))
        rows += w2.T
        lens, nq = [9000, 300, 50000], [5, 300, 40]
        g = torch.Generator().manual_seed(3)
        sc = torch.randn(sum(nq), max(lens), generator=g).to(DEV)
        cu_q = torch.tensor(np.concatenate([[0], np.cumsum(nq)]), dtype=torch.int32, device=DEV)
        dsa.dsa_topk(sc, 2048, torch.tensor(lens, dtype=torch.int32, device=DEV), cu_q=cu_q,
                     max_ctx=max(lens))
        rows += sum(nq)
        torch.cuda.synchronize()
    finally:
        dsa.dsa_set_index_checks(None)
    got = c.cpu().numpy().tolist()
    assert got == [0, 0, 0, rows], got


def test_index_check_counts_planted_faults(dsa):
    """dsa_check_index_rows alone (no attention) on host-built rows with
    planted faults: its counts equal the same counts taken on the host."""
    say("index-row check on planted faults")
    g = np.random.default_rng(9)
    lens = [40, 3000, 700, 5]
    K = 64
    rows = []
    for n in lens:
        keff = min(K, n)
        r = np.sort(g.choice(n, size=keff, replace=False)).astype(np.int32)
        rows.append(np.concatenate([r, np.full(K - keff, -1, np.int32)]))
    idx = np.stack(rows)
    idx[0, 3] = 40          # past p = 39
    idx[1, 10] = -7         # below -1
    idx[1, 20], idx[1, 21] = idx[1, 21], idx[1, 20]   # a descending pair
    idx[2, 0] = -1          # a -1 before positions (and one position fewer)
    idx[3, 5] = 4           # a position in the padding (one more than K_eff = 5)

    def host_counts(full):
        bad = order = wrong = 0
        for t, n in enumerate(lens):
            r = idx[t]
            bad += int(np.sum((r < -1) | (r > n - 1)))
            if full:
                a, b = r[:-1], r[1:]
                order += int(np.sum(((a < 0) & (b >= 0)) | ((a >= 0) & (b >= 0) & (b <= a))))
                wrong += int(np.sum(r >= 0) != min(K, n))
        return [bad, order if full else 0, wrong if full else 0, len(lens)]

    ctx = torch.tensor(lens, dtype=torch.int32, device=DEV)
    d_idx = torch.from_numpy(idx).to(DEV)
    for full in (True, False):
        c = dsa.dsa_check_index_rows(d_idx, ctx, full=full)
        torch.cuda.synchronize()
        got = c.cpu().numpy().tolist()
        assert got == host_counts(full), (full, got, host_counts(full))
        assert got[0] == 2


def test_internal_workspaces_on_a_side_stream(dsa):
    """Calls on a stream that is not the current one, with the binding's own
    workspaces: while they run, the current stream allocates and overwrites
    fresh memory; the results still match the oracle."""
    say("dsa_topk and dsa_sparse_attn on a side stream with internal workspaces")
    side = torch.cuda.Stream()
    n, K = 131072, 2048
    x = _topk_case("relu_like", n, seed=9)
    ctx = torch.tensor([n], dtype=torch.int32)
    w = wl("t", [n], [1], 4, 64, 64, 128, K, seed=25)
    inp = W.make_inputs(w)
    idx_r = _rand_idx([n], [1], K, seed=8)
    d = to_dev(inp)
    xs, cs, ir = x[None].to(DEV).contiguous(), ctx.to(DEV), idx_r.to(DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        pass
    got = dsa.dsa_topk(xs, K, cs, max_ctx=n, stream=side)
    out = dsa.dsa_sparse_attn(d["q"], d["k_cache"], d["v_cache"], ir, d["ctx_len"], d["cu_ctx"],
                              gate=d["gate"], max_ctx=n, stream=side)
    junk = [torch.full((1 << 20,), 7, dtype=torch.int32, device=DEV) for _ in range(8)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    want = oracle.topk(x[None].numpy().astype(np.float32), K, ctx.numpy())
    assert np.array_equal(got.cpu().numpy(), want)
    ref, _ = oracle.sparse_attn(inp["q"], inp["k_cache"], inp["v_cache"], idx=idx_r,
                                gate=inp["gate"], ctx_len=inp["ctx_len"], cu_ctx=inp["cu_ctx"])
    check_out(out, ref, ATOL_BF16)


# --------------------------------------------------------------------------
# Cache append (standalone and fused with the decode layer)
# --------------------------------------------------------------------------

def _append_rows(ctx_lens, n_q):
    """Cache row of every query row: cu_ctx[b] + p."""
    cu = np.concatenate([[0], np.cumsum(ctx_lens)])
    return [int(cu[b] + p) for b, (L, n) in enumerate(zip(ctx_lens, n_q))
            for p in range(L - n, L)]


@pytest.mark.parametrize("key,d_I,lens,nq", [("fp8", 128, [5000, 300, 77], [1, 1, 1]),
                                             ("bf16", 128, [5000, 300, 77], [1, 1, 1]),
                                             ("fp8", 128, [6000, 2500], [40, 130]),
                                             ("fp8", 64, [900, 4000], [3, 1])])
def test_cache_append_bit_exact(dsa, key, d_I, lens, nq):
    say(f"cache append {key} d_I={d_I} lens={lens} nq={nq}")
    w = wl("t", lens, nq, 4 if d_I == 64 else 32, d_I, 64, 128, 64, key_dtype=key, seed=71)
    d = W.make_inputs(w, device=DEV)
    T, L_tot = w.T, sum(lens)
    k_idx_new = W.randn_bf16((T, d_I), 71, "k_idx_new", DEV)
    k_idx_new[0] *= 300.0                      # a row with a large range
    k_idx_new[-1] = 0                          # an all-zero row
    k_new = W.randn_bf16((T, 128), 71, "k_new", DEV)
    v_new = W.randn_bf16((T, 128), 71, "v_new", DEV)
    before = {n: d[n].clone() for n in ("k_idx", "k_cache", "v_cache")}
    ks_before = None if d["k_scale"] is None else d["k_scale"].clone()
    cu_q = None if all(n == 1 for n in nq) else d["cu_q"]
    dsa.dsa_cache_append(d["ctx_len"], d["cu_ctx"], k_idx_cache=d["k_idx"], k_idx_new=k_idx_new,
                         k_scale_cache=d["k_scale"], k_cache=d["k_cache"], k_new=k_new,
                         v_cache=d["v_cache"], v_new=v_new, cu_q=cu_q)
    torch.cuda.synchronize()
    rows = torch.tensor(_append_rows(lens, nq), dtype=torch.int64, device=DEV)
    mask = torch.ones(L_tot, dtype=torch.bool, device=DEV)
    mask[rows] = False
    for n, new in (("k_cache", k_new), ("v_cache", v_new)):
        assert torch.equal(d[n][rows], new)
        assert torch.equal(d[n][mask], before[n][mask])
    if key == "fp8":
        codes, scales = oracle.quantize_e4m3_rows(cpu(k_idx_new))
        assert np.array_equal(d["k_idx"][rows].view(torch.uint8).cpu().numpy(), codes)
        assert np.array_equal(d["k_scale"][rows].cpu().numpy(), scales)
        assert torch.equal(d["k_scale"][mask], ks_before[mask])
        assert torch.equal(d["k_idx"].view(torch.uint8)[mask],
                           before["k_idx"].view(torch.uint8)[mask])
    else:
        assert torch.equal(d["k_idx"][rows], k_idx_new)
        assert torch.equal(d["k_idx"][mask], before["k_idx"][mask])


@pytest.mark.parametrize("key,lens,H_I", [
    ("bf16", [131072], 32),               # deep tiles of two waves; p in the second wave
    ("fp8", [131072, 40000, 23001], 32),  # p in either wave, ragged
    ("bf16", [4096, 70000, 2048, 129], 16),
    ("fp8", [300000, 1 << 20], 32),       # shallow one-wave tiles
])
def test_layer_decode_append_fused(dsa, key, lens, H_I):
    """The fused append-and-decode call leaves the same caches and gives the
    same bits as dsa_cache_append followed by dsa_layer_decode; the result
    is also checked against the oracle on the appended caches."""
    say(f"layer_decode_append {key} lens={lens}")
    w = wl("t", lens, [1] * len(lens), H_I, 128, 64, 128, 2048, key_dtype=key, seed=72,
           plant_frac=0.05 if key == "bf16" else 0.0)
    a = W.make_inputs(w, device=DEV)
    b = {n: (v.clone() if isinstance(v, torch.Tensor) else v) for n, v in a.items()}
    k_idx_new = W.randn_bf16((w.B, 128), 72, "k_idx_new", DEV) * 3
    k_new = W.randn_bf16((w.B, 128), 72, "k_new", DEV)
    v_new = W.randn_bf16((w.B, 128), 72, "v_new", DEV)
    L = max(lens)
    nb = dsa.dsa_layer_decode_workspace_size(w.B, L, w.K, w.Hq, w.D)
    idx_a = torch.empty(w.B, w.K, dtype=torch.int32, device=DEV)
    out_a = dsa.dsa_layer_decode_append(a["q_idx"], a["w"], a["k_idx"], a["k_scale"], a["q"],
                                        a["k_cache"], a["v_cache"], a["gate"], w.K, a["ctx_len"],
                                        a["cu_ctx"], k_idx_new, k_new, v_new, max_ctx=L,
                                        idx_out=idx_a,
                                        ws=torch.full((nb,), 255, dtype=torch.uint8, device=DEV))
    dsa.dsa_cache_append(b["ctx_len"], b["cu_ctx"], k_idx_cache=b["k_idx"], k_idx_new=k_idx_new,
                         k_scale_cache=b["k_scale"], k_cache=b["k_cache"], k_new=k_new,
                         v_cache=b["v_cache"], v_new=v_new)
    idx_b = torch.empty_like(idx_a)
    out_b = dsa.dsa_layer_decode(b["q_idx"], b["w"], b["k_idx"], b["k_scale"], b["q"],
                                 b["k_cache"], b["v_cache"], b["gate"], w.K, b["ctx_len"],
                                 b["cu_ctx"], max_ctx=L, idx_out=idx_b)
    torch.cuda.synchronize()
    for n in ("k_idx", "k_cache", "v_cache"):
        assert torch.equal(a[n].view(torch.uint8), b[n].view(torch.uint8)), n
    if key == "fp8":
        assert torch.equal(a["k_scale"], b["k_scale"])
    assert torch.equal(idx_a, idx_b)
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    if sum(lens) <= 300000:
        cpu_in = {n: cpu(v) if isinstance(v, torch.Tensor) else v for n, v in a.items()}
        _layer_decode_check(dsa, w, cpu_in, a, atol=ATOL_FP8 if key == "fp8" else ATOL_BF16)


def test_layer_decode_append_large_batch_row_sweeps(dsa):
    """1024 sequences: the fused append in the indexer without Top-K reports."""
    say("layer_decode_append, 1024 ragged sequences")
    g = np.random.default_rng(73)
    lens = [int(x) for x in g.integers(300, 3000, size=1024)]
    w = wl("t", lens, [1] * len(lens), 4, 64, 8, 64, 256, key_dtype="fp8", seed=73)
    a = W.make_inputs(w, device=DEV)
    b = {n: (v.clone() if isinstance(v, torch.Tensor) else v) for n, v in a.items()}
    k_idx_new = W.randn_bf16((w.B, 64), 73, "k_idx_new", DEV)
    k_new = W.randn_bf16((w.B, 64), 73, "k_new", DEV)
    v_new = W.randn_bf16((w.B, 64), 73, "v_new", DEV)
    L = max(lens)
    out_a = dsa.dsa_layer_decode_append(a["q_idx"], a["w"], a["k_idx"], a["k_scale"], a["q"],
                                        a["k_cache"], a["v_cache"], a["gate"], w.K, a["ctx_len"],
                                        a["cu_ctx"], k_idx_new, k_new, v_new, max_ctx=L)
    dsa.dsa_cache_append(b["ctx_len"], b["cu_ctx"], k_idx_cache=b["k_idx"], k_idx_new=k_idx_new,
                         k_scale_cache=b["k_scale"], k_cache=b["k_cache"], k_new=k_new,
                         v_cache=b["v_cache"], v_new=v_new)
    out_b = dsa.dsa_layer_decode(b["q_idx"], b["w"], b["k_idx"], b["k_scale"], b["q"],
                                 b["k_cache"], b["v_cache"], b["gate"], w.K, b["ctx_len"],
                                 b["cu_ctx"], max_ctx=L)
    torch.cuda.synchronize()
    for n in ("k_idx", "k_cache", "v_cache"):
        assert torch.equal(a[n].view(torch.uint8), b[n].view(torch.uint8)), n
    assert torch.equal(a["k_scale"], b["k_scale"])
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
