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
from tests.parity import (ATOL_BF16, ATOL_FP8, check_index_row, check_out, check_set_band, cpu,
                          positions)

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


@pytest.mark.parametrize("H_I,d_I,key,lens,nq", [
    (16, 128, "bf16", [3000], [200]),
    (32, 128, "bf16", [2500, 700], [70, 33]),
    (4, 64, "bf16", [1200], [130]),
    (16, 128, "fp8", [2100], [90]),
])
def test_index_scores_prefill(dsa, H_I, d_I, key, lens, nq):
    say(f"index_scores prefill H_I={H_I} {key} lens={lens} nq={nq}")
    w = wl("t", lens, nq, H_I, d_I, 8, 64, 64, key_dtype=key, seed=12)
    inp = W.make_inputs(w)
    d = to_dev(inp)
    s = torch.full((w.T, max(lens)), float("nan"), device=DEV)
    dsa.dsa_index_scores(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["ctx_len"], d["cu_ctx"],
                         cu_q=d["cu_q"], max_ctx=max(lens), scores=s)
    torch.cuda.synchronize()
    ref = oracle.index_scores(inp["q_idx"], inp["w"], inp["k_idx"], inp["k_scale"],
                              ctx_len=inp["ctx_len"], cu_q=inp["cu_q"], cu_ctx=inp["cu_ctx"])
    got = s.cpu().numpy().astype(np.float64)
    for t, p in enumerate(positions(lens, nq)):
        err = np.abs(got[t, :p + 1] - ref[t, :p + 1])
        assert np.all(err <= _score_tol(ref[t, :p + 1])), f"row {t}: max err {err.max():.3g}"
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
    cnt = torch.zeros(5, dtype=torch.int32, device=DEV)
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
    assert c[1] == len(lens)


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


def test_hybrid_step_swa_layers_then_dsa_layer(dsa):
    """One decode step of the 5:1 hybrid at a small ragged shape: two
    sliding-window layers (own K/V caches, ungated, through the prepared-call
    path the bench uses) and one Gated DSA layer, each against the oracle."""
    say("hybrid step: 2 SWA layers (window 128) + 1 DSA layer, ragged batch")
    lens = [130, 5000, 777]
    w = wl("t", lens, [1] * 3, 16, 128, 64, 128, 256, seed=41)
    inp = W.make_inputs(w)
    d = to_dev(inp)
    ntot = sum(lens)
    for i in range(2):
        q = W.randn_bf16((3, 64, 128), 41, f"swa{i}_q")
        k = W.randn_bf16((ntot, 128), 41, f"swa{i}_k")
        v = W.randn_bf16((ntot, 128), 41, f"swa{i}_v")
        out = torch.empty(3, 64, 128, dtype=torch.bfloat16, device=DEV)
        call = dsa.prepare_sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), None, d["ctx_len"],
                                       d["cu_ctx"], max(lens), out, window=128)
        call()
        call()  # re-issued: same result
        torch.cuda.synchronize()
        ref, _ = oracle.sparse_attn(q, k, v, window=128, ctx_len=inp["ctx_len"],
                                    cu_ctx=inp["cu_ctx"])
        check_out(out, ref, ATOL_BF16)
    _layer_decode_check(dsa, w, inp, d)


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def _layer_decode_check(dsa, w, inp_cpu, d, seqs=None, atol=ATOL_BF16):
    B = w.B
    idx = torch.empty(B, w.K, dtype=torch.int32, device=DEV)
    out = dsa.dsa_layer_decode(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["q"], d["k_cache"],
                               d["v_cache"], d["gate"], w.K, d["ctx_len"], d["cu_ctx"],
                               max_ctx=max(w.ctx_lens), idx_out=idx)
    torch.cuda.synchronize()
    idx_c = idx.cpu().numpy()
    seqs = range(B) if seqs is None else seqs
    ndiff = 0
    for b in seqs:
        L = w.ctx_lens[b]
        r0 = int(sum(w.ctx_lens[:b]))
        ks = None if inp_cpu["k_scale"] is None else inp_cpu["k_scale"][r0:r0 + L]
        s_ref = oracle.index_scores(inp_cpu["q_idx"][b:b + 1], inp_cpu["w"][b:b + 1],
                                    inp_cpu["k_idx"][r0:r0 + L], ks,
                                    ctx_len=np.array([L], np.int32))[0]
        sel = check_index_row(idx_c[b], L - 1, w.K)
        ndiff += check_set_band(sel, s_ref, L - 1, w.K)
        ref, _ = oracle.sparse_attn(inp_cpu["q"][b:b + 1], inp_cpu["k_cache"][r0:r0 + L],
                                    inp_cpu["v_cache"][r0:r0 + L], idx=idx_c[b:b + 1],
                                    gate=inp_cpu["gate"][b:b + 1],
                                    ctx_len=np.array([L], np.int32))
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
    say("layer_decode determinism")
    w = W.decode_128k()
    inp = W.make_inputs(w)
    d = to_dev(inp)
    outs = []
    for _ in range(3):
        idx = torch.empty(1, w.K, dtype=torch.int32, device=DEV)
        o = dsa.dsa_layer_decode(d["q_idx"], d["w"], d["k_idx"], None, d["q"], d["k_cache"],
                                 d["v_cache"], d["gate"], w.K, d["ctx_len"], d["cu_ctx"],
                                 max_ctx=w.ctx_lens[0], idx_out=idx)
        outs.append((o.clone(), idx.clone()))
    torch.cuda.synchronize()
    for o, i in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(i, outs[0][1])


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
    out = dsa.dsa_layer_decode(inp["q_idx"], inp["w"], inp["k_idx"], inp["k_scale"], inp["q"],
                               inp["k_cache"], inp["v_cache"], inp["gate"], w.K, inp["ctx_len"],
                               inp["cu_ctx"], max_ctx=L, idx_out=idx)
    torch.cuda.synchronize()
    idx_c = idx.cpu().numpy()
    for b in samp:
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


def _layer_prefill_check(dsa, w, inp, d, rows=None):
    idx = torch.empty(w.T, w.K, dtype=torch.int32, device=DEV)
    out = dsa.dsa_layer_prefill(d["q_idx"], d["w"], d["k_idx"], d["k_scale"], d["q"],
                                d["k_cache"], d["v_cache"], d["gate"], w.K, d["cu_q"],
                                d["ctx_len"], d["cu_ctx"], max_q=max(w.n_q),
                                max_ctx=max(w.ctx_lens), idx_out=idx)
    torch.cuda.synchronize()
    idx_c = idx.cpu().numpy()
    pos = positions(w.ctx_lens, w.n_q)
    seq_of = np.repeat(np.arange(w.B), w.n_q)
    rows = range(w.T) if rows is None else rows
    cu_ctx = np.concatenate([[0], np.cumsum(w.ctx_lens)])
    for t in rows:
        b, p = int(seq_of[t]), pos[t]
        r0 = int(cu_ctx[b])
        ks = None if inp["k_scale"] is None else cpu(inp["k_scale"][r0:r0 + p + 1])
        s_ref = oracle.index_scores_at(cpu(inp["q_idx"][t]), cpu(inp["w"][t]),
                                       cpu(inp["k_idx"][r0:r0 + p + 1]), ks)
        sel = check_index_row(idx_c[t], p, w.K)
        check_set_band(sel, s_ref, p, w.K)
        rr = torch.from_numpy(sel.astype(np.int64)) + r0
        dev = inp["k_cache"].device
        ref, _ = oracle.sparse_attn(cpu(inp["q"][t:t + 1]), cpu(inp["k_cache"][rr.to(dev)]),
                                    cpu(inp["v_cache"][rr.to(dev)]),
                                    idx=np.arange(len(sel), dtype=np.int32)[None],
                                    gate=cpu(inp["gate"][t:t + 1]),
                                    ctx_len=np.array([len(sel)], np.int32))
        check_out(out[t:t + 1], ref, ATOL_BF16 if inp["k_scale"] is None else ATOL_FP8)


def test_layer_prefill_small(dsa):
    say("layer_prefill 2 sequences, short and long rows")
    w = wl("t", [6000, 2500], [300, 2500], 16, 128, 64, 128, 2048, seed=41)
    inp = W.make_inputs(w)
    _layer_prefill_check(dsa, w, inp, to_dev(inp), rows=list(range(0, w.T, 37)) + [w.T - 1])


def test_layer_prefill_tiny_shape(dsa):
    say("layer_prefill tiny shape (4x64 indexer, 8 heads x 64)")
    w = wl("t", [4096], [64], 4, 64, 8, 64, 256, seed=42)
    inp = W.make_inputs(w)
    _layer_prefill_check(dsa, w, inp, to_dev(inp))


def test_layer_prefill_8k_chunk_sampled(dsa):
    say("layer_prefill 8192 queries on a 131072-token context (sampled rows)")
    w = W.prefill_8k()
    inp = W.make_inputs(w, device=DEV)
    _layer_prefill_check(dsa, w, inp, inp, rows=[0, 1, 2047, 4096, 8190, 8191])


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
