"""Pins of the fp64 CPU oracle against things other than itself.

Every pin below comes from a library routine, a closed form, an identity of
the mathematics, a hand-derived example (tests/golden) or brute force on
tiny inputs.  Together they cover each term of the score, the selection
rule, the softmax attention and the gate, so that a dropped term, a wrong
sign, a wrong index or a transposed operand fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def seq(ctx, nq=1):
    return dict(ctx_len=np.array([ctx], np.int32), cu_q=np.array([0, nq], np.int32))


# --------------------------------------------------------------------------
# Input decoding
# --------------------------------------------------------------------------

def test_bf16_widening_matches_torch_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3fn_decoding_matches_torch_and_ocp_spec():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}          # only S.1111.111 is NaN
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0       # largest finite, no infinities
    assert got[0x01] == 2.0 ** -9                           # smallest subnormal
    assert got[0x08] == 2.0 ** -6                           # smallest normal


# --------------------------------------------------------------------------
# Indexer score
# --------------------------------------------------------------------------

def test_hand_example_scores_and_topk():
    g = json.load(open(os.path.join(GOLD, "hand_example_scores_topk.json")))
    q = bf16([g["q_idx"]])
    w = bf16([g["w"]])
    k = bf16(g["k_idx"])
    s = oracle.index_scores(q, w, k, **seq(4))
    assert s[0].tolist() == g["scores"]
    for K, want in g["topk"].items():
        assert oracle.topk(s, int(K), np.array([4], np.int32))[0].tolist() == want
    # two new queries at positions 2 and 3: the first sees positions 0..2 only
    q2 = torch.cat([q, q])
    w2 = torch.cat([w, w])
    s2 = oracle.index_scores(q2, w2, k, ctx_len=np.array([4], np.int32),
                             cu_q=np.array([0, 2], np.int32))
    assert s2[0, :3].tolist() == g["causal_p2_scores"] and np.isnan(s2[0, 3])
    idx = oracle.topk(s2, 2, np.array([4], np.int32), cu_q=np.array([0, 2], np.int32))
    assert idx[0].tolist() == g["causal_p2_top2"]


def test_one_hot_query_gives_relu_of_key_coordinate():
    rng = np.random.default_rng(0)
    k = bf16(rng.standard_normal((50, 8)))
    for d in range(8):
        q = torch.zeros(1, 1, 8, dtype=torch.bfloat16)
        q[0, 0, d] = 1
        s = oracle.index_scores(q, bf16([[1.0]]), k, **seq(50))
        assert np.array_equal(s[0], np.maximum(k[:, d].double().numpy(), 0.0))


def test_relu_identities_against_library_dot():
    # One head, unit weight: s(q) - s(-q) = q.k and s(q) + s(-q) = |q.k| (ReLU(x) -/+ ReLU(-x)).
    rng = np.random.default_rng(1)
    k = bf16(rng.standard_normal((200, 64)))
    q = bf16(rng.standard_normal((1, 1, 64)))
    sp = oracle.index_scores(q, bf16([[1.0]]), k, **seq(200))[0]
    sm = oracle.index_scores(-q, bf16([[1.0]]), k, **seq(200))[0]
    dot = k.double().numpy() @ q[0, 0].double().numpy()
    np.testing.assert_allclose(sp - sm, dot, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sp + sm, np.abs(dot), rtol=1e-12, atol=1e-12)


def test_head_weights_combine_linearly_and_per_head():
    # s(w) = sum_h w_h * s(e_h), and s(e_h) is the single-head score of head h.
    rng = np.random.default_rng(2)
    H, d, L = 4, 16, 64
    k = bf16(rng.standard_normal((L, d)))
    q = bf16(rng.standard_normal((1, H, d)))
    w = bf16(rng.uniform(-1, 1, (1, H)))
    s = oracle.index_scores(q, w, k, **seq(L))[0]
    parts = []
    for h in range(H):
        e = torch.zeros(1, H, dtype=torch.bfloat16)
        e[0, h] = 1
        sh = oracle.index_scores(q, e, k, **seq(L))[0]
        single = oracle.index_scores(q[:, h:h + 1], bf16([[1.0]]), k, **seq(L))[0]
        assert np.array_equal(sh, single)
        dot = k.double().numpy() @ q[0, h].double().numpy()
        np.testing.assert_allclose(sh, np.maximum(dot, 0), rtol=1e-12, atol=1e-12)
        parts.append(sh)
    want = sum(float(w[0, h]) * parts[h] for h in range(H))
    np.testing.assert_allclose(s, want, rtol=1e-12, atol=1e-12)


def test_scores_do_not_depend_on_position():
    # No RoPE in the indexer: permuting cache rows permutes the scores exactly.
    rng = np.random.default_rng(3)
    k = bf16(rng.standard_normal((40, 16)))
    q = bf16(rng.standard_normal((1, 4, 16)))
    w = bf16(rng.uniform(0, 1, (1, 4)))
    perm = rng.permutation(40)
    s = oracle.index_scores(q, w, k, **seq(40))[0]
    sp = oracle.index_scores(q, w, k[perm], **seq(40))[0]
    assert np.array_equal(sp, s[perm])


def test_fp8_scale_multiplies_before_relu():
    rng = np.random.default_rng(4)
    L = 30
    k8 = torch.from_numpy(rng.standard_normal((L, 16)).astype(np.float32)).to(torch.float8_e4m3fn)
    q = bf16(rng.standard_normal((1, 2, 16)))
    w = bf16([[1.0, 0.5]])
    one = oracle.index_scores(q, w, k8, k_scale=np.ones(L, np.float32), **seq(L))[0]
    c = rng.uniform(0.5, 2.0, L).astype(np.float32)
    sc = oracle.index_scores(q, w, k8, k_scale=c, **seq(L))[0]
    np.testing.assert_allclose(sc, c.astype(np.float64) * one, rtol=1e-12, atol=1e-12)
    # negative scale: ReLU acts on the dequantised product, so the score is
    # the ReLU of the opposite dot product, not -1 times the positive-scale one
    neg = oracle.index_scores(q, w, k8, k_scale=-np.ones(L, np.float32), **seq(L))[0]
    kd = k8.double().numpy()
    want = sum(float(w[0, h]) * np.maximum(-(kd @ q[0, h].double().numpy()), 0) for h in range(2))
    np.testing.assert_allclose(neg, want, rtol=1e-12, atol=1e-12)
    # dequantised keys equal bf16 keys holding the same values
    s16 = oracle.index_scores(q, w, k8.float().to(torch.bfloat16), **seq(L))[0]
    assert np.array_equal(one, s16)


def test_shared_weight_row_and_packed_batch():
    rng = np.random.default_rng(5)
    lens = [7, 12, 5]
    kk = bf16(rng.standard_normal((sum(lens), 8)))
    q = bf16(rng.standard_normal((3, 2, 8)))
    w = bf16(rng.uniform(0, 1, (2,)))
    s = oracle.index_scores(q, w, kk, ctx_len=np.array(lens, np.int32), w_ld=0)
    off = 0
    for b, L in enumerate(lens):
        sb = oracle.index_scores(q[b:b + 1], w[None], kk[off:off + L], **seq(L))[0]
        assert np.array_equal(s[b, :L], sb)
        assert np.all(np.isnan(s[b, L:]))
        off += L


# --------------------------------------------------------------------------
# Top-K selection
# --------------------------------------------------------------------------

def brute_force_topk(s, K):
    """Unique subset S with |S| = min(K, n) such that every member beats every
    non-member under (score desc, position asc); found by enumeration."""
    n = len(s)
    keff = min(K, n)
    found = []
    for S in itertools.combinations(range(n), keff):
        Sset = set(S)
        ok = all((s[i] > s[j]) or (s[i] == s[j] and i < j)
                 for i in S for j in range(n) if j not in Sset)
        if ok:
            found.append(list(S))
    assert len(found) == 1
    return found[0] + [-1] * (K - keff)


def test_topk_matches_subset_enumeration_with_ties():
    rng = np.random.default_rng(6)
    vals = np.array([0.0, -0.0, 1.0, 2.0, 2.0, -1.0, 0.5])
    for trial in range(60):
        n = int(rng.integers(1, 10))
        s = rng.choice(vals, n)
        for K in range(1, n + 3):
            got = oracle.topk(s[None].astype(np.float64), K, np.array([n], np.int32))[0]
            assert got.tolist() == brute_force_topk(s.tolist(), K), (s, K)
            got32 = oracle.topk(s[None].astype(np.float32), K, np.array([n], np.int32))[0]
            assert got32.tolist() == got.tolist()


def test_topk_special_cases():
    L = 100
    ctx = np.array([L], np.int32)
    eq = np.full((1, L), 3.5)
    assert oracle.topk(eq, 10, ctx)[0].tolist() == list(range(10))
    ramp = np.arange(L, dtype=np.float64)[None]
    assert oracle.topk(ramp, 10, ctx)[0].tolist() == list(range(90, 100))
    assert oracle.topk(ramp, 128, ctx)[0].tolist() == list(range(100)) + [-1] * 28
    z = np.zeros((1, 4))
    z[0, 0] = -0.0
    z[0, 2] = -0.0
    assert oracle.topk(z, 2, np.array([4], np.int32))[0].tolist() == [0, 1]


def test_topk_certificate_on_random_rows():
    rng = np.random.default_rng(7)
    L, K = 5000, 256
    s = np.round(rng.standard_normal((3, L)) * 20) / 4     # many exact ties
    idx = oracle.topk(s, K, np.array([L], np.int32), cu_q=np.array([0, 3], np.int32))
    for r in range(3):
        p = L - 3 + r
        sel = idx[r]
        assert np.all(np.diff(sel) > 0) and sel.min() >= 0 and sel.max() <= p
        mask = np.zeros(p + 1, bool)
        mask[sel] = True
        worst_in = min(sel, key=lambda j: (s[r, j], -j))
        rest = np.nonzero(~mask)[0]
        best_out = max(rest, key=lambda j: (s[r, j], -j))
        assert (s[r, worst_in] > s[r, best_out]) or (
            s[r, worst_in] == s[r, best_out] and worst_in < best_out)


def test_topk_ratio_at_one_million_context():
    # "roughly 500x" fewer elements at a 1,048,576 context with K = 2048
    assert (1 << 20) // 2048 == 512


# --------------------------------------------------------------------------
# Gated sparse attention
# --------------------------------------------------------------------------

def test_hand_example_attention():
    g = json.load(open(os.path.join(GOLD, "hand_example_attention.json")))
    q = bf16([g["q"]])
    kc = bf16(g["k_rows"])
    vc = bf16(g["v_rows"])
    gate = bf16([g["gate"]])
    out, lse = oracle.sparse_attn(q, kc, vc, idx=np.array([[0, 1]], np.int32), gate=gate,
                                  sm_scale=g["sm_scale"], ctx_len=np.array([2], np.int32))
    np.testing.assert_allclose(out[0], g["out"], rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(lse[0], g["lse"], rtol=1e-15)


def _attn_case(rng, L, Hq, D, T=1):
    q = bf16(rng.standard_normal((T, Hq, D)))
    kc = bf16(rng.standard_normal((L, D)))
    vc = bf16(rng.standard_normal((L, D)))
    g = bf16(rng.standard_normal((T, Hq, D)))
    return q, kc, vc, g


def test_full_selection_equals_dense_attention_sdpa():
    # K >= context: sparse attention is full causal attention (library SDPA).
    rng = np.random.default_rng(8)
    L, Hq, D, T = 37, 4, 16, 5
    q, kc, vc, g = _attn_case(rng, L, Hq, D, T)
    cu_q = np.array([0, T], np.int32)
    idx = np.tile(np.arange(64, dtype=np.int32), (T, 1))
    for t in range(T):
        idx[t, L - T + t + 1:] = -1
    out, lse = oracle.sparse_attn(q, kc, vc, idx=idx, gate=g, ctx_len=np.array([L], np.int32),
                                  cu_q=cu_q)
    qd = q.double().permute(1, 0, 2)[None]                     # [1, Hq, T, D]
    kd = kc.double()[None, None].expand(1, Hq, L, D)
    vd = vc.double()[None, None].expand(1, Hq, L, D)
    mask = torch.zeros(T, L, dtype=torch.bool)
    for t in range(T):
        mask[t, :L - T + t + 1] = True
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=mask)
    ref = ref[0].permute(1, 0, 2) * torch.sigmoid(g.double())
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-12)
    logits = (qd @ kd.transpose(-1, -2)) / math.sqrt(D)
    logits = logits.masked_fill(~mask, -math.inf)
    ref_lse = torch.logsumexp(logits, -1)[0].T
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(9)
    L, Hq, D = 50, 3, 8
    q, kc, vc, g = _attn_case(rng, L, Hq, D)
    ctx = np.array([L], np.int32)
    sig = torch.sigmoid(g.double()).numpy()[0]
    # K = 1: output is the gated value row
    out, _ = oracle.sparse_attn(q, kc, vc, idx=np.array([[17]], np.int32), gate=g, ctx_len=ctx)
    np.testing.assert_allclose(out[0], sig * vc[17].double().numpy()[None], rtol=1e-15)
    # q = 0: mean of the selected rows
    sel = np.array([[3, 9, 30, 44, -1, -1]], np.int32)
    out, _ = oracle.sparse_attn(torch.zeros_like(q), kc, vc, idx=sel, ctx_len=ctx)
    np.testing.assert_allclose(out[0], np.tile(vc[[3, 9, 30, 44]].double().numpy().mean(0),
                                               (Hq, 1)), rtol=1e-13)
    # constant value rows: output is that row whatever the weights
    vconst = vc.clone()
    vconst[:] = vc[5]
    out, _ = oracle.sparse_attn(q, kc, vconst, idx=sel, gate=g, ctx_len=ctx)
    np.testing.assert_allclose(out[0], sig * vc[5].double().numpy()[None], rtol=1e-13)
    # order of the index list does not matter; -1 entries are ignored
    a, la = oracle.sparse_attn(q, kc, vc, idx=sel, ctx_len=ctx)
    b, lb = oracle.sparse_attn(q, kc, vc, idx=np.array([[-1, 44, 3, -1, 30, 9]], np.int32),
                               ctx_len=ctx)
    np.testing.assert_allclose(a, b, rtol=1e-14)
    # convex combination: each coordinate within the selected rows' range
    rows = vc[[3, 9, 30, 44]].double().numpy()
    assert np.all(a[0] <= rows.max(0) + 1e-12) and np.all(a[0] >= rows.min(0) - 1e-12)
    # a very large gate leaves the ungated output
    big = torch.full_like(g, 60.0)
    c, _ = oracle.sparse_attn(q, kc, vc, idx=sel, gate=big, ctx_len=ctx)
    np.testing.assert_allclose(c, a, rtol=1e-15)
    # explicit scale: logits scaled by 2/sqrt(D) equal q doubled at the default scale
    d1, _ = oracle.sparse_attn(q, kc, vc, idx=sel, ctx_len=ctx, sm_scale=2 / math.sqrt(D))
    d2, _ = oracle.sparse_attn((q.float() * 2).to(torch.bfloat16), kc, vc, idx=sel, ctx_len=ctx)
    np.testing.assert_allclose(d1, d2, rtol=1e-13)


def test_sliding_window_equals_explicit_indices_and_dense_tail():
    rng = np.random.default_rng(10)
    L, Hq, D, W = 300, 2, 16, 128
    q, kc, vc, _ = _attn_case(rng, L, Hq, D)
    ctx = np.array([L], np.int32)
    win, lw = oracle.sparse_attn(q, kc, vc, window=W, ctx_len=ctx)
    idx = np.arange(L - W, L, dtype=np.int32)[None]
    exp_, le = oracle.sparse_attn(q, kc, vc, idx=idx, ctx_len=ctx)
    np.testing.assert_allclose(win, exp_, rtol=1e-15)
    qd = q.double().permute(1, 0, 2)[None]
    kd = kc[L - W:].double()[None, None].expand(1, Hq, W, D)
    vd = vc[L - W:].double()[None, None].expand(1, Hq, W, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd)[0].permute(1, 0, 2)
    np.testing.assert_allclose(win, ref.numpy(), rtol=1e-10, atol=1e-12)
    # a window longer than the context covers positions 0..p only
    short, _ = oracle.sparse_attn(q, kc[:50], vc[:50], window=W, ctx_len=np.array([50], np.int32))
    full, _ = oracle.sparse_attn(q, kc[:50], vc[:50], idx=np.arange(50, dtype=np.int32)[None],
                                 ctx_len=np.array([50], np.int32))
    np.testing.assert_allclose(short, full, rtol=1e-15)


def test_layer_with_k_at_least_context_is_gated_dense_attention():
    rng = np.random.default_rng(11)
    L, H, d, Hq, D, K = 40, 4, 16, 4, 16, 64
    qi = bf16(rng.standard_normal((1, H, d)))
    w = bf16(rng.uniform(0, 1, (1, H)))
    ki = bf16(rng.standard_normal((L, d)))
    q, kc, vc, g = _attn_case(rng, L, Hq, D)
    r = oracle.layer(qi, w, ki, None, q, kc, vc, g, K, np.array([L], np.int32))
    assert r["idx"][0].tolist() == list(range(L)) + [-1] * (K - L)
    qd = q.double().permute(1, 0, 2)[None]
    kd = kc.double()[None, None].expand(1, Hq, L, D)
    vd = vc.double()[None, None].expand(1, Hq, L, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd)[0].permute(1, 0, 2)
    ref = ref * torch.sigmoid(g.double())
    np.testing.assert_allclose(r["out"], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_layer_selection_is_topk_of_its_own_scores():
    rng = np.random.default_rng(12)
    L, H, d, Hq, D, K = 500, 4, 16, 2, 16, 32
    qi = bf16(rng.standard_normal((1, H, d)))
    w = bf16(rng.uniform(0, 1, (1, H)))
    ki = bf16(rng.standard_normal((L, d)))
    q, kc, vc, g = _attn_case(rng, L, Hq, D)
    r = oracle.layer(qi, w, ki, None, q, kc, vc, g, K, np.array([L], np.int32))
    s = oracle.index_scores(qi, w, ki, **seq(L))
    assert np.array_equal(r["scores"], s)
    assert np.array_equal(r["idx"], oracle.topk(s, K, np.array([L], np.int32)))
    out, _ = oracle.sparse_attn(q, kc, vc, idx=r["idx"], gate=g, ctx_len=np.array([L], np.int32))
    assert np.array_equal(r["out"], out)


# --------------------------------------------------------------------------
# Cache-append quantisation (bf16 key row -> E4M3FN codes + fp32 scale)
# --------------------------------------------------------------------------

def _torch_codes(k_bf16, sigma):
    """Reference rounding: torch's own fp32 -> float8_e4m3fn cast (round to
    nearest, ties to even) of y = x / sigma clamped to the format's range."""
    y = k_bf16.float() / torch.from_numpy(sigma)[:, None]
    y = y.clamp(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_quantize_matches_torch_rounding_on_varied_rows():
    rng = np.random.default_rng(20)
    rows = [rng.standard_normal(128),
            rng.standard_normal(128) * 1e-3,
            rng.standard_normal(128) * 300.0,
            np.where(rng.random(128) < 0.05, 40.0, 1.0) * rng.standard_normal(128),  # outliers
            rng.standard_normal(128) * 1e-30,                                          # tiny scale
            np.linspace(-1, 1, 128),
            np.zeros(128)]
    k = bf16(np.stack(rows))
    codes, sigma = oracle.quantize_e4m3_rows(k)
    amax = np.abs(k.float().numpy()).max(1)
    want_sigma = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    assert np.array_equal(sigma, want_sigma)
    assert np.array_equal(codes, _torch_codes(k, sigma))
    # the largest magnitude of each non-zero row lands on +-448 (code 0x7E / 0xFE)
    for r in range(len(rows) - 1):
        i = int(np.abs(k[r].float().numpy()).argmax())
        assert codes[r, i] & 0x7F == 0x7E
    assert np.all(codes[-1] == 0) and sigma[-1] == 1.0


def test_quantize_ties_go_to_even_codes():
    # amax = 448 gives sigma = 1 exactly, so y = x: each value below sits
    # exactly halfway between two E4M3FN neighbours (hand-computed codes)
    vals = [448.0, 1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, 5 * 2.0 ** -10, -1.0625, 17.0,
            2.0 ** -6 * (1 + 1 / 16), 0.0]
    want = [0x7E,           # 448 = 1.75 * 2^8
            0x38,           # 1.0625: between 1.0 (0x38) and 1.125 (0x39) -> even 0x38
            0x3A,           # 1.1875: between 1.125 (0x39) and 1.25 (0x3A) -> even 0x3A
            0x02,           # 1.5 * 2^-9 -> 2 * 2^-9 (even)
            0x00,           # 0.5 * 2^-9 -> 0 (even)
            0x02,           # 2.5 * 2^-9 -> 2 * 2^-9 (even)
            0xB8,           # -1.0625 -> -1.0
            0x58,           # 17 between 16 (0x58) and 18 (0x59) -> even 0x58
            0x08,           # 2^-6 * 1.0625 between 2^-6 (0x08) and 2^-6*1.125 (0x09) -> 0x08
            0x00]
    row = np.zeros(64)
    row[:len(vals)] = vals
    codes, sigma = oracle.quantize_e4m3_rows(bf16(row[None]))
    assert sigma[0] == 1.0
    assert codes[0, :len(vals)].tolist() == want
    assert np.array_equal(codes, _torch_codes(bf16(row[None]), sigma))


def test_quantize_error_within_half_a_code_step():
    rng = np.random.default_rng(21)
    k = bf16(rng.standard_normal((50, 64)) * rng.uniform(0.01, 100, (50, 1)))
    codes, sigma = oracle.quantize_e4m3_rows(k)
    y = np.clip(k.float().numpy() / sigma[:, None], -448, 448)
    dec = oracle.e4m3_to_f64(codes.ravel()).reshape(codes.shape)
    a = np.abs(y)
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 1e-30))) - 3))
    assert np.all(np.abs(dec - y) <= step / 2 + 1e-12)


# --------------------------------------------------------------------------
# E4M3FN query heads with a per-(query, head) scale
# --------------------------------------------------------------------------

def _fp8(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)


def test_fp8_queries_with_unit_scale_equal_bf16_queries_of_the_same_values():
    # every E4M3FN value is a bf16 value: torch's own widening gives the bf16 twin
    rng = np.random.default_rng(30)
    q8 = _fp8(rng.standard_normal((3, 4, 16)) * 4)
    k = bf16(rng.standard_normal((60, 16)))
    w = bf16(rng.uniform(0, 1, (3, 4)))
    kw = dict(ctx_len=np.array([60], np.int32), cu_q=np.array([0, 3], np.int32))
    s8 = oracle.index_scores(q8, w, k, q_scale=np.ones((3, 4), np.float32), **kw)
    s16 = oracle.index_scores(q8.to(torch.bfloat16), w, k, **kw)
    assert np.array_equal(s8, s16, equal_nan=True)


def test_fp8_query_scale_is_linear_per_head_and_acts_before_the_relu():
    rng = np.random.default_rng(31)
    H, d, L = 4, 16, 50
    q8 = _fp8(rng.standard_normal((1, H, d)) * 3)
    k8 = _fp8(rng.standard_normal((L, d)))
    ks = rng.uniform(0.5, 2.0, L).astype(np.float32)
    w = bf16(rng.uniform(0, 1, (1, H)))
    one = np.ones((1, H), np.float32)
    base = oracle.index_scores(q8, w, k8, ks, q_scale=one, **seq(L))[0]
    # a common positive factor on every head scales the score
    c = np.float32(1.75)
    np.testing.assert_allclose(oracle.index_scores(q8, w, k8, ks, q_scale=one * c, **seq(L))[0],
                               c * base, rtol=1e-13, atol=0)
    # one head's scale acts like that head's weight (a positive power of two,
    # exact in the bf16 weight too)
    rho = one.copy()
    rho[0, 2] = 4.0
    w2 = w.float().clone()
    w2[0, 2] *= 4.0
    np.testing.assert_allclose(oracle.index_scores(q8, w, k8, ks, q_scale=rho, **seq(L))[0],
                               oracle.index_scores(q8, bf16(w2.numpy()), k8, ks, q_scale=one,
                                                   **seq(L))[0], rtol=1e-13, atol=0)
    # a negative query scale flips the sign inside the ReLU (closed form)
    neg = oracle.index_scores(q8, w, k8, ks, q_scale=-one, **seq(L))[0]
    dots = k8.double().numpy() @ q8[0].double().numpy().T          # [L, H]
    want = (np.maximum(-(ks[:, None].astype(np.float64) * dots), 0) *
            w[0].double().numpy()[None]).sum(1)
    np.testing.assert_allclose(neg, want, rtol=1e-12, atol=1e-12)


def test_fp8_queries_and_keys_match_a_dense_fp64_formula():
    # brute force through numpy on decoded values (an independent code path)
    rng = np.random.default_rng(32)
    T, H, d, L = 3, 4, 64, 40
    q8 = _fp8(rng.standard_normal((T, H, d)) * 2)
    rho = rng.uniform(0.25, 4.0, (T, H)).astype(np.float32)
    k8 = _fp8(rng.standard_normal((L, d)))
    ks = rng.uniform(0.5, 2.0, L).astype(np.float32)
    w = bf16(rng.uniform(0, 1, (T, H)))
    s = oracle.index_scores(q8, w, k8, ks, q_scale=rho, ctx_len=np.array([L], np.int32),
                            cu_q=np.array([0, T], np.int32))
    qd, kd = q8.double().numpy(), k8.double().numpy()
    dots = np.einsum("thd,jd->thj", qd, kd)
    x = rho.astype(np.float64)[:, :, None] * ks.astype(np.float64)[None, None, :] * dots
    ref = (w.double().numpy()[:, :, None] * np.maximum(x, 0)).sum(1)
    for t in range(T):
        p = L - T + t
        np.testing.assert_allclose(s[t, :p + 1], ref[t, :p + 1], rtol=1e-12, atol=1e-12)
        assert np.all(np.isnan(s[t, p + 1:]))
