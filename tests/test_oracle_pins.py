"""Pins of the CPU oracle against what the source page and the mathematics fix.

The method ("MiniMax goes sparse: decoding M3's attention from a single diagram", §1 Step 1
and Step 2) has no printed worked example, so the oracle is pinned by:
  * a hand-derived example in the diagram's shape (tests/golden/diagram_shape_example.json);
  * the dense special case: keeping every block must reproduce dense GQA attention
    (torch SDPA, float64), since attention runs on the real K/V;
  * brute-force enumeration of every k-subset on tiny inputs, and numpy's stable argsort;
  * the linearity identity: <mean query, mean key> = mean of the token-level scores;
  * a masked dense softmax as a second route to sparse attention over the selected blocks;
  * closed forms: one visible token, q = 0, constant V, weights summing to 1;
  * invariances: page permutation, power-of-two query scaling;
  * prefill: k >= candidates gives dense causal attention; k = 0 gives the diagonal block
    alone (local causal attention).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import make_decode_case, make_prefill_case, storage, round_to_bf16
from helpers import as_f64, dense_gqa, decode_inputs, logical_kv, prefill_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "diagram_shape_example.json")


# ----------------------------------------------------------------------------- golden example
def _golden_inputs(dtype):
    g = json.load(open(GOLDEN))
    Hq, Hkv, D, P, N = g["Hq"], g["Hkv"], g["D"], g["P"], g["N"]
    nb = N // P
    k = np.zeros((nb, Hkv, P, D), np.float32)
    v = np.zeros((nb, Hkv, P, D), np.float32)
    for grp in range(Hkv):
        for t in range(N):
            k[t // P, grp, t % P] = g["k"][str(grp)][t]
            v[t // P, grp, t % P] = g["v"][str(grp)][t]
    q = np.array(g["q"], np.float32)[None]
    table = np.arange(nb, dtype=np.int32)[None]
    return g, dict(q=storage(q, dtype), k_pool=storage(k, dtype), v_pool=storage(v, dtype),
                   block_table=table, seq_lens=np.array([N], np.int32), Hq=Hq, Hkv=Hkv,
                   scale=g["scale"], P=P)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_golden_diagram_example(dtype):
    g, kw = _golden_inputs(dtype)
    ex = g["expected"]
    r1 = oracle.decode(top_k=1, want_weights=True, **kw)
    np.testing.assert_array_equal(r1["scores"][0], np.array(ex["scores"], np.float64))
    np.testing.assert_array_equal(r1["idx"][0], np.array(ex["k1"]["idx"]))
    np.testing.assert_allclose(r1["o"][0], np.array(ex["k1"]["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(r1["lse"][0], np.array(ex["k1"]["lse"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(r1["w"][0].sum(axis=1), 1.0, atol=1e-15)
    r2 = oracle.decode(top_k=2, **kw)
    np.testing.assert_array_equal(r2["idx"][0], np.array(ex["k2"]["idx"]))
    np.testing.assert_allclose(r2["o"][0, 0], ex["k2"]["o_head0"], atol=1e-14)
    np.testing.assert_allclose(r2["lse"][0, 0], ex["k2"]["lse_head0"], atol=1e-14)


# ----------------------------------------------------------------------------- top-k
def _brute_force_topk(s, k):
    """The unique k-subset S with: for i in S, j not in S, s_i > s_j or (s_i == s_j and i < j)."""
    n = len(s)
    keff = min(k, n)
    winners = []
    for S in itertools.combinations(range(n), keff):
        inside = set(S)
        if all((s[i] > s[j]) or (s[i] == s[j] and i < j)
               for i in inside for j in range(n) if j not in inside):
            winners.append(list(S))
    assert len(winners) == 1
    return winners[0] + [-1] * (k - keff)


@pytest.mark.parametrize("seed", range(40))
def test_topk_brute_force(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(1, 13))
    k = int(r.integers(1, 6))
    # integer-valued scores make ties frequent; half the cases also include -0.0 and +0.0
    s = r.integers(-3, 4, size=n).astype(np.float64)
    if seed % 2:
        s[s == 0] = -0.0
        s[::3] = np.where(s[::3] == 0, 0.0, s[::3])
    got = oracle.topk(s, k)
    assert list(got) == _brute_force_topk(list(s), k)


@pytest.mark.parametrize("seed", range(10))
def test_topk_matches_stable_argsort(seed):
    r = np.random.default_rng(100 + seed)
    n = int(r.integers(50, 5000))
    k = int(r.integers(1, 200))
    s = np.round(r.standard_normal(n), 2)  # rounded: many ties
    want = np.sort(np.argsort(-s, kind="stable")[:min(k, n)])
    got = oracle.topk(s, k)
    np.testing.assert_array_equal(got[:len(want)], want)
    assert np.all(got[len(want):] == -1)


def test_topk_special_cases():
    np.testing.assert_array_equal(oracle.topk(np.full(10, 3.5), 4), [0, 1, 2, 3])
    s = np.array([0.1, 0.9, -2.0, 0.9, 0.5])
    np.testing.assert_array_equal(oracle.topk(s, 1), [1])          # first argmax
    np.testing.assert_array_equal(oracle.topk(s, 8), [0, 1, 2, 3, 4, -1, -1, -1])  # k >= nb
    np.testing.assert_array_equal(oracle.topk(np.array([-0.0, 0.0]), 1), [0])  # -0 == +0


# ----------------------------------------------------------------------------- stage 1
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scores_equal_mean_token_scores(dtype):
    """<mean of the group's queries, mean of the block's keys> = mean over (head, token) of
    <q_h, k_t>: token-level scores, pooled, computed with numpy matmul."""
    c = make_decode_case(B=2, Hq=6, Hkv=2, lens=[1000, 130], top_k=4, dtype=dtype, seed=3)
    r = oracle.decode(**decode_inputs(c))
    G = c.Hq // c.Hkv
    for b in range(c.B):
        N = int(c.seq_lens[b])
        K = as_f64(storage(logical_kv(c.k_pool, c.block_table, b, N), dtype))
        qb = as_f64(storage(c.q[b], dtype))
        for g in range(c.Hkv):
            tok = qb[g * G:(g + 1) * G] @ K[:, g, :].T   # [G][N]
            nb = (N + c.P - 1) // c.P
            want = [tok[:, j * c.P:min(N, (j + 1) * c.P)].mean() for j in range(nb)]
            np.testing.assert_allclose(r["scores"][b, g, :nb], want, rtol=1e-12, atol=1e-12)
            assert np.all(np.isneginf(r["scores"][b, g, nb:]))


def test_scores_scale_exactly_with_power_of_two_query():
    c = make_decode_case(B=1, Hq=8, Hkv=2, lens=[777], top_k=5, dtype="f32", seed=4)
    kw = decode_inputs(c)
    r = oracle.decode(**kw)
    kw2 = dict(kw, q=(kw["q"] * np.float32(8.0)).astype(np.float32))
    r2 = oracle.decode(**kw2)
    np.testing.assert_array_equal(r2["scores"], r["scores"] * 8.0)
    np.testing.assert_array_equal(r2["idx"], r["idx"])


# ----------------------------------------------------------------------------- stage 2
@pytest.mark.parametrize("dtype,lens,Hq,Hkv", [("f32", [640], 6, 2), ("bf16", [1000, 64, 1], 8, 2),
                                               ("f32", [4096], 8, 1), ("bf16", [333], 32, 8)])
def test_all_blocks_equals_dense_gqa(dtype, lens, Hq, Hkv):
    """k >= nb: the sparse path must be dense GQA attention over the real K/V."""
    nbmax = max((n + 63) // 64 for n in lens)
    c = make_decode_case(B=len(lens), Hq=Hq, Hkv=Hkv, lens=lens, top_k=nbmax + 3, dtype=dtype, seed=5)
    r = oracle.decode(**decode_inputs(c))
    for b, N in enumerate(lens):
        K = as_f64(storage(logical_kv(c.k_pool, c.block_table, b, N), dtype))
        V = as_f64(storage(logical_kv(c.v_pool, c.block_table, b, N), dtype))
        o, lse = dense_gqa(as_f64(storage(c.q[b], dtype)), K, V, c.scale)
        np.testing.assert_allclose(r["o"][b], o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(r["lse"][b], lse, rtol=1e-12, atol=1e-12)
        nb = (N + 63) // 64
        assert list(r["idx"][b, 0, :nb]) == list(range(nb))


@pytest.mark.parametrize("seed", range(4))
def test_sparse_equals_masked_dense(seed):
    """Attention over the gathered blocks == dense softmax with every unselected token masked."""
    c = make_decode_case(B=2, Hq=6, Hkv=2, lens=[1500, 700], top_k=5, dtype="bf16", seed=seed,
                         plant=("count", 2), permute=True)
    r = oracle.decode(want_weights=True, **decode_inputs(c))
    G = c.Hq // c.Hkv
    for b in range(c.B):
        N = int(c.seq_lens[b])
        K = as_f64(storage(logical_kv(c.k_pool, c.block_table, b, N), "bf16"))
        V = as_f64(storage(logical_kv(c.v_pool, c.block_table, b, N), "bf16"))
        qb = as_f64(storage(c.q[b], "bf16"))
        for g in range(c.Hkv):
            sel = r["idx"][b, g]
            assert len(set(sel[sel >= 0])) == (sel >= 0).sum() and np.all(np.diff(sel[sel >= 0]) > 0)
            mask = np.isin(np.arange(N) // c.P, sel[sel >= 0])
            o, lse = dense_gqa(qb[g * G:(g + 1) * G], K[:, g:g + 1], V[:, g:g + 1], c.scale, mask=mask)
            np.testing.assert_allclose(r["o"][b, g * G:(g + 1) * G], o, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(r["lse"][b, g * G:(g + 1) * G], lse, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(r["w"][b, g * G:(g + 1) * G].sum(axis=1), 1.0, atol=1e-13)


def test_closed_forms():
    # one visible token: o is that value row, lse the single logit
    c = make_decode_case(B=1, Hq=4, Hkv=1, lens=[1], top_k=1, dtype="f32", seed=6)
    r = oracle.decode(**decode_inputs(c))
    v0 = c.v_pool[c.block_table[0, 0], 0, 0].astype(np.float64)
    k0 = c.k_pool[c.block_table[0, 0], 0, 0].astype(np.float64)
    for h in range(4):
        np.testing.assert_array_equal(r["o"][0, h], v0)
        np.testing.assert_allclose(r["lse"][0, h], c.scale * float(c.q[0, h].astype(np.float64) @ k0), atol=1e-14)
    # q = 0: uniform weights over the selected tokens -> o = their mean, lse = ln(count)
    c = make_decode_case(B=1, Hq=4, Hkv=2, lens=[900], top_k=3, dtype="f32", seed=7)
    kw = decode_inputs(c)
    kw["q"] = np.zeros_like(kw["q"])
    r = oracle.decode(**kw)
    V = logical_kv(c.v_pool, c.block_table, 0, 900).astype(np.float64)
    for g in range(2):
        sel = r["idx"][0, g]
        assert list(sel) == [0, 1, 2]  # all scores are 0: ties break to the lowest indices
        toks = np.concatenate([np.arange(j * 64, min(900, j * 64 + 64)) for j in sel])
        np.testing.assert_allclose(r["o"][0, 2 * g], V[toks, g].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(r["lse"][0, 2 * g], math.log(len(toks)), atol=1e-13)
    # constant V: o = that constant whatever the weights
    c = make_decode_case(B=1, Hq=8, Hkv=2, lens=[2000], top_k=4, dtype="bf16", seed=8)
    kw = decode_inputs(c)
    kw["v_pool"] = storage(np.full(c.v_pool.shape, 1.75, np.float32), "bf16")
    r = oracle.decode(**kw)
    np.testing.assert_allclose(r["o"], 1.75, rtol=1e-14)


def test_empty_sequence():
    c = make_decode_case(B=2, Hq=4, Hkv=2, lens=[0, 100], top_k=2, dtype="f32", seed=9)
    r = oracle.decode(**decode_inputs(c))
    assert np.all(r["idx"][0] == -1)
    assert np.all(r["o"][0] == 0) and np.all(np.isneginf(r["lse"][0]))
    assert np.all(np.isfinite(r["o"][1]))


def test_page_permutation_invariance():
    a = make_decode_case(B=2, Hq=8, Hkv=2, lens=[3000, 1234], top_k=6, dtype="bf16", seed=10)
    kw = decode_inputs(a)
    r1 = oracle.decode(**kw)
    perm = np.random.default_rng(0).permutation(a.num_pages)   # new page id of old page p = perm[p]
    k2 = np.empty_like(kw["k_pool"]); k2[perm] = kw["k_pool"]
    v2 = np.empty_like(kw["v_pool"]); v2[perm] = kw["v_pool"]
    t2 = np.where(a.block_table >= 0, perm[np.maximum(a.block_table, 0)], -1).astype(np.int32)
    r2 = oracle.decode(**dict(kw, k_pool=k2, v_pool=v2, block_table=t2))
    for key in ("scores", "idx", "o", "lse"):
        np.testing.assert_array_equal(r1[key], r2[key])


def test_idx_override_and_padding():
    c = make_decode_case(B=1, Hq=4, Hkv=1, lens=[500], top_k=4, dtype="f32", seed=11)
    kw = decode_inputs(c)
    forced = np.array([[[7, 2, -1, 99]]], np.int32)     # unsorted, padded, out-of-range entry
    r = oracle.decode(idx_in=forced, **kw)
    mask = np.isin(np.arange(500) // 64, [2, 7])
    K = logical_kv(c.k_pool, c.block_table, 0, 500).astype(np.float64)
    V = logical_kv(c.v_pool, c.block_table, 0, 500).astype(np.float64)
    o, lse = dense_gqa(c.q[0].astype(np.float64), K, V, c.scale, mask=mask)
    np.testing.assert_allclose(r["o"][0], o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["lse"][0], lse, rtol=1e-12)


def test_precomputed_summaries_agree():
    c = make_decode_case(B=3, Hq=8, Hkv=2, lens=[1000, 64, 65], top_k=3, dtype="bf16", seed=12, permute=True)
    kw = decode_inputs(c)
    S = oracle.summaries(k_pool=kw["k_pool"], block_table=c.block_table, seq_lens=c.seq_lens,
                         Hkv=c.Hkv, D=c.D, P=c.P)
    r1 = oracle.decode(**kw)
    r2 = oracle.decode(summaries_in=S, **kw)
    for key in ("scores", "idx", "o", "lse"):
        np.testing.assert_array_equal(r1[key], r2[key])
    # partial block: mean over the valid tokens only (the padded slots hold a large constant)
    last = as_f64(kw["k_pool"][c.block_table[2, 1], :, :1, :]).mean(axis=1)
    np.testing.assert_allclose(S[2, 1], last, rtol=1e-15)


@pytest.mark.parametrize("name,shape", [("small_fp32", dict(B=1, Hq=8, Hkv=1, lens=[4096], top_k=16, dtype="f32", plant=("count", 3))),
                                        ("small_bf16", dict(B=2, Hq=32, Hkv=8, lens=[8192, 8192], top_k=32, dtype="bf16", plant=("frac", 0.01)))])
def test_planted_blocks_are_found(name, shape):
    """Sanity of the input recipe: blocks lifted along the group's query direction rank high."""
    c = make_decode_case(seed=13, **shape)
    r = oracle.decode(**decode_inputs(c))
    hit = tot = 0
    for (b, g), blocks in c.planted.items():
        hit += len(set(blocks) & set(r["idx"][b, g]))
        tot += len(blocks)
    assert hit / tot >= 0.9


# ----------------------------------------------------------------------------- prefill
@pytest.mark.parametrize("past_len,T,dtype", [(256, 128, "f32"), (128, 100, "bf16"), (0, 130, "f32")])
def test_prefill_all_blocks_equals_dense_causal(past_len, T, dtype):
    c = make_prefill_case(Hq=8, Hkv=2, past_len=past_len, T=T, top_k=64, dtype=dtype, seed=14)
    kw = prefill_inputs(c)
    r = oracle.prefill(**kw)
    N = past_len + T
    Kc = logical_kv(c.k_pool, c.block_table, 0, past_len) if past_len else np.zeros((0, 2, 128), np.float32)
    Vc = logical_kv(c.v_pool, c.block_table, 0, past_len) if past_len else np.zeros((0, 2, 128), np.float32)
    K = as_f64(storage(np.concatenate([Kc, c.k_new]), dtype))
    V = as_f64(storage(np.concatenate([Vc, c.v_new]), dtype))
    mask = np.arange(N)[None, :] <= (past_len + np.arange(T))[:, None]
    o, lse = dense_gqa(as_f64(kw["q"]), K, V, c.scale, mask=mask)
    np.testing.assert_allclose(r["o"], o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=1e-12, atol=1e-12)
    ntiles = (T + 63) // 64
    for tau in range(ntiles):
        d = past_len // 64 + tau
        assert list(r["idx"][tau, 0, :d + 1]) == list(range(d + 1))


def test_prefill_k0_is_local_causal():
    c = make_prefill_case(Hq=4, Hkv=1, past_len=192, T=150, top_k=0, dtype="f32", seed=15)
    r = oracle.prefill(**prefill_inputs(c))
    for tau in range(3):
        rows = slice(tau * 64, min(150, tau * 64 + 64))
        n = rows.stop - rows.start
        K = c.k_new[rows].astype(np.float64)
        V = c.v_new[rows].astype(np.float64)
        mask = np.tril(np.ones((n, n), bool))
        o, lse = dense_gqa(c.q[rows].astype(np.float64), K, V, c.scale, mask=mask)
        np.testing.assert_allclose(r["o"][rows], o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(r["lse"][rows], lse, rtol=1e-12, atol=1e-12)
        assert r["idx"][tau, 0, 0] == 3 + tau


def test_prefill_selection_and_tile_scores():
    """Tile scores = mean over the tile's (row, head, token) scores; selection = oracle top-k over
    the blocks before the diagonal, then the diagonal appended; sampled tiles agree with a full run."""
    c = make_prefill_case(Hq=8, Hkv=2, past_len=640, T=200, top_k=3, dtype="bf16", seed=16)
    kw = prefill_inputs(c)
    r = oracle.prefill(**kw)
    part = oracle.prefill(tiles=(1, 3), **kw)
    np.testing.assert_array_equal(part["o"][64:192], r["o"][64:192])
    np.testing.assert_array_equal(part["idx"][1:3], r["idx"][1:3])
    G = 4
    K = as_f64(storage(np.concatenate([logical_kv(c.k_pool, c.block_table, 0, 640), c.k_new]), "bf16"))
    q = as_f64(kw["q"])
    for tau in range(4):
        rows = slice(tau * 64, min(200, tau * 64 + 64))
        d = 10 + tau
        for g in range(2):
            tok = q[rows, g * G:(g + 1) * G].reshape(-1, 128) @ K[:, g].T
            want = np.array([tok[:, j * 64:(j + 1) * 64].mean() for j in range(d)])
            np.testing.assert_allclose(r["scores"][tau, g, :d], want, rtol=1e-12, atol=1e-12)
            sel = oracle.topk(want, 3)
            assert list(r["idx"][tau, g]) == list(sel) + [d]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_idx_override(dtype):
    """The prefill oracle's route that attends over given lists (the GPU tests fall back to it when
    a GPU list differs from the oracle's inside the tie band):
      * its own lists fed back reproduce the plain run bit for bit;
      * a list with one selected block dropped, a -1 entry and entries above the tile's diagonal
        block equals dense causal attention (torch SDPA, float64) whose mask keeps only the listed
        blocks at or below the diagonal: those above it are ignored, the diagonal (the last slot,
        position top_k) still counts."""
    past, T, k, Hkv, G = 640, 150, 4, 2, 4
    c = make_prefill_case(Hq=Hkv * G, Hkv=Hkv, past_len=past, T=T, top_k=k, dtype=dtype, seed=31)
    kw = prefill_inputs(c)
    r = oracle.prefill(**kw)
    r2 = oracle.prefill(idx_in=r["idx"], **kw)
    np.testing.assert_array_equal(r2["o"], r["o"])
    np.testing.assert_array_equal(r2["lse"], r["lse"])
    ntiles = (T + 63) // 64
    idx = r["idx"].copy()
    for tau in range(ntiles):
        d = past // 64 + tau
        for g in range(Hkv):
            assert idx[tau, g, k] == d                     # k_eff = k here: the diagonal is the last slot
            idx[tau, g, (tau + g) % k] = -1                # one selected block dropped
            idx[tau, g, (tau + g + 1) % k] = d + 1 + g     # above the diagonal: ignored
    rt = oracle.prefill(idx_in=idx, **kw)
    N = past + T
    K = as_f64(storage(np.concatenate([logical_kv(c.k_pool, c.block_table, 0, past), c.k_new]), dtype))
    V = as_f64(storage(np.concatenate([logical_kv(c.v_pool, c.block_table, 0, past), c.v_new]), dtype))
    q = as_f64(kw["q"])
    for tau in range(ntiles):
        rows = np.arange(tau * 64, min(T, tau * 64 + 64))
        d = past // 64 + tau
        for g in range(Hkv):
            keep = [j for j in idx[tau, g] if 0 <= j <= d]
            assert len(keep) == k - 1                      # k - 2 selected blocks + the diagonal
            mask = np.isin(np.arange(N) // 64, keep)[None, :] & (np.arange(N)[None, :] <= (past + rows)[:, None])
            heads = slice(g * G, (g + 1) * G)
            o, lse = dense_gqa(q[rows][:, heads], K[:, g:g + 1], V[:, g:g + 1], c.scale, mask=mask)
            np.testing.assert_allclose(rt["o"][rows][:, heads], o, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(rt["lse"][rows][:, heads], lse, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- index branch (R8)
# The pages' literal Step 1: single-head index keys shared by every group, one index query per
# group, token scores, Block Max Pool, TopK (oracle.select_index).
def _index_case(lens=(200, 64, 131), Hkv=3, Di=16, seed=5):
    rng = np.random.default_rng(seed)
    nb = [(n + 63) // 64 for n in lens]
    mb = max(nb) + 1
    num_pages = sum(nb) + 3
    perm = rng.permutation(num_pages)
    table = np.full((len(lens), mb), -1, np.int32)
    p = 0
    for b, n in enumerate(nb):
        for j in range(n):
            table[b, j] = perm[p]
            p += 1
    q = rng.standard_normal((len(lens), Hkv, Di)).astype(np.float32)
    ik = rng.standard_normal((num_pages, 64, Di)).astype(np.float32)
    return q, ik, table, np.array(lens, np.int32)


def _token_value(b, t):
    return np.float32(10.0 * math.sin(1.7 * t + 0.3 * b) + 0.01 * t)


def test_index_max_pool_closed_form():
    """q_idx[b][g] = (g + 1) e0, so a token scores (g + 1) * K_idx[t][0] and a block scores
    (g + 1) * max of dim 0 over its valid tokens; slots past the length hold a huge dim 0."""
    q, ik, table, lens = _index_case()
    B, Hkv, Di = q.shape
    q[:] = 0.0
    q[:, :, 0] = np.arange(1, Hkv + 1, dtype=np.float32)[None, :]
    ik[:, :, 0] = 1.0e6                                   # never a valid token's value
    for b in range(B):
        for t in range(int(lens[b])):
            ik[table[b, t // 64], t % 64, 0] = _token_value(b, t)
    r = oracle.select_index(q_idx=q, index_keys=ik, block_table=table, seq_lens=lens, top_k=2)
    for b in range(B):
        n = int(lens[b])
        nb = (n + 63) // 64
        for g in range(Hkv):
            for j in range(table.shape[1]):
                if j < nb:
                    want = (g + 1) * max(float(_token_value(b, t)) for t in range(64 * j, min(n, 64 * j + 64)))
                    assert r["scores"][b, g, j] == want
                else:
                    assert r["scores"][b, g, j] == -np.inf


def test_index_reduces_to_mean_pool_for_constant_blocks():
    """When every valid token of a block carries the same index key, max pool == mean pool: the
    mean-pool route (orc_decode's summaries and scores with G = 1, q = q_idx, every group's keys
    = the index keys) gives the same scores and the same lists."""
    q, ik, table, lens = _index_case(Hkv=2, Di=8)
    for b in range(len(lens)):
        for j in range((int(lens[b]) + 63) // 64):
            ik[table[b, j], :, :] = ik[table[b, j], 0, :]
    k = 3
    r = oracle.select_index(q_idx=q, index_keys=ik, block_table=table, seq_lens=lens, top_k=k)
    Hkv, Di = q.shape[1], q.shape[2]
    kp = np.ascontiguousarray(np.repeat(ik[:, None], Hkv, axis=1))      # [pages][Hkv][64][Di]
    d = oracle.decode(q=q, k_pool=kp, v_pool=kp, block_table=table, seq_lens=lens, Hq=Hkv, Hkv=Hkv,
                      top_k=k, scale=1.0)
    for b in range(len(lens)):
        nb = (int(lens[b]) + 63) // 64
        assert np.array_equal(r["scores"][b, :, :nb], d["scores"][b, :, :nb])
    assert np.array_equal(r["idx"], d["idx"])


def test_index_invariances():
    """Reordering the tokens of a full block, or moving blocks to other pages (table updated),
    changes no score and no list; bf16 storage equals its exact float32 upcast."""
    q, ik, table, lens = _index_case(lens=(256, 320))
    base = oracle.select_index(q_idx=q, index_keys=ik, block_table=table, seq_lens=lens, top_k=3)
    ik2 = ik.copy()
    rng = np.random.default_rng(1)
    for page in range(ik.shape[0]):
        ik2[page] = ik[page][rng.permutation(64)]          # every block of these sequences is full
    r2 = oracle.select_index(q_idx=q, index_keys=ik2, block_table=table, seq_lens=lens, top_k=3)
    assert np.array_equal(base["scores"], r2["scores"]) and np.array_equal(base["idx"], r2["idx"])
    perm = rng.permutation(ik.shape[0])
    ik3 = np.empty_like(ik)
    ik3[perm] = ik
    table3 = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
    r3 = oracle.select_index(q_idx=q, index_keys=ik3, block_table=table3, seq_lens=lens, top_k=3)
    assert np.array_equal(base["scores"], r3["scores"]) and np.array_equal(base["idx"], r3["idx"])
    qb, ikb = storage(q, "bf16"), storage(ik, "bf16")
    rb = oracle.select_index(q_idx=qb, index_keys=ikb, block_table=table, seq_lens=lens, top_k=3)
    ru = oracle.select_index(q_idx=round_to_bf16(q), index_keys=round_to_bf16(ik), block_table=table,
                             seq_lens=lens, top_k=3)
    assert np.array_equal(rb["scores"], ru["scores"]) and np.array_equal(rb["idx"], ru["idx"])


def test_index_query_scaling_and_group_order():
    """A positive factor on an index query scales every token score and hence every block maximum
    by that factor (exactly for a power of two) and keeps the lists; permuting the groups of the
    index queries permutes the score rows and the lists the same way."""
    q, ik, table, lens = _index_case(lens=(200, 64, 131, 700), Hkv=4, Di=16, seed=17)
    base = oracle.select_index(q_idx=q, index_keys=ik, block_table=table, seq_lens=lens, top_k=3)
    fin = np.isfinite(base["scores"])
    r4 = oracle.select_index(q_idx=q * np.float32(4.0), index_keys=ik, block_table=table, seq_lens=lens, top_k=3)
    assert np.array_equal(r4["scores"][fin], 4.0 * base["scores"][fin])
    assert np.array_equal(np.isfinite(r4["scores"]), fin) and np.array_equal(r4["idx"], base["idx"])
    c = np.array([0.25, 8.0, 2.0, 0.5], np.float32)[None, :, None]    # a different factor per group
    rc = oracle.select_index(q_idx=q * c, index_keys=ik, block_table=table, seq_lens=lens, top_k=3)
    assert np.array_equal(rc["scores"][fin], (base["scores"] * c.astype(np.float64))[fin])
    assert np.array_equal(rc["idx"], base["idx"])
    perm = np.array([2, 0, 3, 1])
    rp = oracle.select_index(q_idx=np.ascontiguousarray(q[:, perm]), index_keys=ik, block_table=table, seq_lens=lens,
                             top_k=3)
    assert np.array_equal(rp["scores"], base["scores"][:, perm]) and np.array_equal(rp["idx"], base["idx"][:, perm])


def test_index_planted_token_and_bad_page():
    """A single token planted along group 0's index query makes its block group 0's best block,
    scoring exactly that token's score; a bad page id scores -inf and is never kept."""
    q, ik, table, lens = _index_case(lens=(64 * 9,), Hkv=2, Di=8, seed=9)
    u = q[0, 0] / np.linalg.norm(q[0, 0])
    ik[table[0, 5], 17] = (40.0 * u).astype(np.float32)
    table[0, 2] = 10_000                                  # out of range: never read
    r = oracle.select_index(q_idx=q, index_keys=ik, block_table=table, seq_lens=lens, top_k=8)
    want = float(np.dot(q[0, 0].astype(np.float64), ik[table[0, 5], 17].astype(np.float64)))
    assert r["scores"][0, 0, 5] == pytest.approx(want, rel=1e-15)
    assert np.argmax(r["scores"][0, 0]) == 5
    assert r["scores"][0, 0, 2] == -np.inf and r["scores"][0, 1, 2] == -np.inf
    assert 2 not in r["idx"][0, 0] and 2 not in r["idx"][0, 1]


# ----------------------------------------------------------------------------- forced blocks (R9)
# Optional sink / local blocks: the first keep_sink and the last keep_local candidates are always
# kept and count toward k_eff; the rest of the list is the usual top-k of the other candidates.
def _brute_force_forced(s, k, sink, local):
    """The unique k_eff-subset S that holds F = {j < sink} U {j >= n - local} and where every
    i in S \\ F beats every candidate j outside S: s_i > s_j, or s_i == s_j and i < j."""
    n = len(s)
    keff = min(k, n)
    F = {j for j in range(n) if j < sink or j >= n - local}
    winners = []
    for S in itertools.combinations(range(n), keff):
        inside = set(S)
        if not F <= inside:
            continue
        if all((s[i] > s[j]) or (s[i] == s[j] and i < j)
               for i in inside - F for j in range(n) if j not in inside):
            winners.append(list(S))
    assert len(winners) == 1
    return winners[0] + [-1] * (k - keff)


@pytest.mark.parametrize("seed", range(40))
def test_forced_topk_brute_force(seed):
    r = np.random.default_rng(500 + seed)
    n = int(r.integers(1, 12))
    sink, local = int(r.integers(0, 3)), int(r.integers(0, 3))
    k = sink + local + int(r.integers(0, 4))
    if k == 0:
        k = 1
    s = r.integers(-3, 4, size=n).astype(np.float64)   # frequent ties
    got = oracle.topk(s, k, keep_sink=sink, keep_local=local)
    assert list(got) == _brute_force_forced(list(s), k, sink, local), (n, k, sink, local)


@pytest.mark.parametrize("seed", range(6))
def test_forced_topk_equals_plain_topk_with_forced_scores_raised(seed):
    """Raising the forced blocks' scores above every other score (they tie among themselves, so
    the index order keeps them all) and taking the plain top-k gives the same list."""
    r = np.random.default_rng(600 + seed)
    n = int(r.integers(20, 3000))
    sink, local = int(r.integers(0, 4)), int(r.integers(0, 4))
    k = sink + local + int(r.integers(0, 100))
    k = max(k, 1)
    s = np.round(r.standard_normal(n), 2)
    raised = s.copy()
    raised[:sink] = np.inf
    raised[max(0, n - local):] = np.inf
    np.testing.assert_array_equal(oracle.topk(s, k, keep_sink=sink, keep_local=local), oracle.topk(raised, k))


def test_forced_topk_special_cases():
    s = np.array([9.0, 1.0, 8.0, 7.0, 0.5, 2.0])
    np.testing.assert_array_equal(oracle.topk(s, 2, keep_sink=1, keep_local=1), [0, 5])   # exactly F
    np.testing.assert_array_equal(oracle.topk(s, 3, keep_sink=1, keep_local=1), [0, 2, 5])  # + best other
    np.testing.assert_array_equal(oracle.topk(s, 3, keep_local=2), [0, 4, 5])
    np.testing.assert_array_equal(oracle.topk(s, 9, keep_sink=2, keep_local=2), [0, 1, 2, 3, 4, 5, -1, -1, -1])
    np.testing.assert_array_equal(oracle.topk(s[:1], 2, keep_sink=1, keep_local=1), [0, -1])  # F overlaps
    with pytest.raises(RuntimeError):
        oracle.topk(s, 1, keep_sink=1, keep_local=1)                  # F does not fit in k


def test_decode_forced_local_block_is_local_attention():
    """k = 1 with the last block forced: every head attends exactly the last (partial) block."""
    c = make_decode_case(B=2, Hq=4, Hkv=2, lens=[1000, 130], top_k=1, dtype="f32", seed=31, permute=True)
    r = oracle.decode(keep_local=1, **decode_inputs(c))
    G = 2
    for b in range(c.B):
        N = int(c.seq_lens[b])
        nb = (N + 63) // 64
        K = logical_kv(c.k_pool, c.block_table, b, N).astype(np.float64)
        V = logical_kv(c.v_pool, c.block_table, b, N).astype(np.float64)
        mask = np.arange(N) >= (nb - 1) * 64
        for g in range(c.Hkv):
            assert list(r["idx"][b, g]) == [nb - 1]
            o, lse = dense_gqa(c.q[b, g * G:(g + 1) * G].astype(np.float64), K[:, g:g + 1], V[:, g:g + 1], c.scale,
                               mask=mask)
            np.testing.assert_allclose(r["o"][b, g * G:(g + 1) * G], o, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(r["lse"][b, g * G:(g + 1) * G], lse, rtol=1e-12, atol=1e-12)


def test_decode_forced_blocks_join_the_selection():
    """sink + local forced, k = 5: the list is {0, nb-1} plus the plain top-3 of the other blocks'
    scores (the scores themselves do not change)."""
    c = make_decode_case(B=1, Hq=8, Hkv=2, lens=[3000], top_k=5, dtype="bf16", seed=32, plant=("count", 3))
    kw = decode_inputs(c)
    plain = oracle.decode(**kw)
    r = oracle.decode(keep_sink=1, keep_local=1, **kw)
    np.testing.assert_array_equal(r["scores"], plain["scores"])
    nb = (3000 + 63) // 64
    for g in range(c.Hkv):
        s = plain["scores"][0, g, :nb]
        others = oracle.topk(s[1:nb - 1], 3) + 1
        assert list(r["idx"][0, g]) == sorted([0, nb - 1] + list(others))


def test_prefill_forced_sink_block():
    """k = 1 with block 0 forced: each tile with cached blocks attends block 0 plus its diagonal
    block (causal); the first tile of a chunk starting at 0 has no candidate, so only its diagonal."""
    c = make_prefill_case(Hq=4, Hkv=1, past_len=256, T=130, top_k=1, dtype="f32", seed=33)
    r = oracle.prefill(keep_sink=1, **prefill_inputs(c))
    K = np.concatenate([logical_kv(c.k_pool, c.block_table, 0, 256), c.k_new]).astype(np.float64)
    V = np.concatenate([logical_kv(c.v_pool, c.block_table, 0, 256), c.v_new]).astype(np.float64)
    for tau in range(3):
        rows = np.arange(tau * 64, min(130, tau * 64 + 64))
        d = 4 + tau
        assert list(r["idx"][tau, 0]) == [0, d]
        pos = 256 + rows
        t = np.arange(K.shape[0])
        mask = ((t[None, :] < 64) | (t[None, :] >= d * 64)) & (t[None, :] <= pos[:, None])
        o, lse = dense_gqa(c.q[rows].astype(np.float64), K, V, c.scale, mask=mask)
        np.testing.assert_allclose(r["o"][rows], o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(r["lse"][rows], lse, rtol=1e-12, atol=1e-12)
    c0 = make_prefill_case(Hq=4, Hkv=1, past_len=0, T=100, top_k=1, dtype="f32", seed=34)
    r0 = oracle.prefill(keep_sink=1, **prefill_inputs(c0))
    assert list(r0["idx"][0, 0]) == [0, -1] and list(r0["idx"][1, 0]) == [0, 1]


def test_prefill_forced_local_block():
    """keep_local = 1: the block just before each tile's diagonal is kept."""
    c = make_prefill_case(Hq=8, Hkv=2, past_len=640, T=200, top_k=3, dtype="bf16", seed=35)
    kw = prefill_inputs(c)
    plain = oracle.prefill(**kw)
    r = oracle.prefill(keep_local=1, **kw)
    for tau in range(4):
        d = 10 + tau
        for g in range(2):
            s = plain["scores"][tau, g, :d]
            want = sorted(list(oracle.topk(s[:d - 1], 2)) + [d - 1])
            assert list(r["idx"][tau, g]) == want + [d]


def test_index_branch_forced_blocks():
    q, ik, table, lens = _index_case()
    kw = dict(q_idx=q, index_keys=ik, block_table=table, seq_lens=lens)
    plain = oracle.select_index(top_k=3, **kw)
    r = oracle.select_index(top_k=3, keep_sink=1, keep_local=1, **kw)
    for b in range(len(lens)):
        nb = (int(lens[b]) + 63) // 64
        for g in range(r["idx"].shape[1]):
            want = oracle.topk(plain["scores"][b, g, :nb], 3, keep_sink=1, keep_local=1)
            np.testing.assert_array_equal(r["idx"][b, g], want)
            assert 0 in r["idx"][b, g] and nb - 1 in r["idx"][b, g]


# ----------------------------------------------------------------------------- bf16 summaries (R10)
# Optional bf16 summary pool: a summary is its block's mean rounded once to bf16, ties to even.
def _one_block_pool(values, Hkv=1, D=128):
    """fp32 pool of one page whose first len(values) tokens hold the given per-token vectors."""
    n = len(values)
    k = np.zeros((1, Hkv, 64, D), np.float32)
    k[0, :, :n, :] = np.asarray(values, np.float32)[None]
    return k, np.zeros((1, 1), np.int32), np.array([n], np.int32)


def test_bf16_summary_of_one_token_is_ieee_rounding():
    """n = 1: the summary is the key itself, so R10 is fp32 -> bf16 round-to-nearest-even, which
    torch's conversion computes; ties (low half exactly 0x8000) are included."""
    r = np.random.default_rng(70)
    x = r.standard_normal(128).astype(np.float32) * np.float32(3.0)
    bits = x.view(np.uint32)
    bits[:32] = (bits[:32] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # exact ties, odd and even
    bits[32:40] = (bits[32:40] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    bits[40:48] = (bits[40:48] & np.uint32(0xFFFF0000)) | np.uint32(0x8001)
    x = bits.view(np.float32)
    k, table, lens = _one_block_pool([x])
    S = oracle.summaries(k_pool=k, block_table=table, seq_lens=lens, Hkv=1, D=128, P=64, summary_dtype="bf16")
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(S[0, 0, 0], want)


def test_bf16_summary_rounds_the_exact_mean_ties_to_even():
    """Means that fall exactly halfway between two bf16 values round to the even one."""
    h = 2.0 ** -8
    rows = [np.full(128, 1.0), np.full(128, 1.0), np.full(128, 1.0 + 3 * h)]        # mean 1 + 2^-8
    rows2 = [np.full(128, 1.0 + 2 * h), np.full(128, 1.0 + 4 * h)]                   # mean 1 + 3*2^-8
    for vals, mean, want in ((rows, 1.0 + h, 1.0), (rows2, 1.0 + 3 * h, 1.0 + 4 * h)):
        k, table, lens = _one_block_pool(vals)
        S = oracle.summaries(k_pool=k, block_table=table, seq_lens=lens, Hkv=1, D=128, P=64, summary_dtype="bf16")
        exact = oracle.summaries(k_pool=k, block_table=table, seq_lens=lens, Hkv=1, D=128, P=64)
        np.testing.assert_array_equal(exact[0, 0, 0], np.full(128, mean))   # the tie itself
        np.testing.assert_array_equal(S[0, 0, 0], np.full(128, want))


def test_bf16_summaries_are_the_rounded_means():
    c = make_decode_case(B=2, Hq=8, Hkv=2, lens=[1000, 130], top_k=4, dtype="bf16", seed=71, permute=True)
    kw = dict(k_pool=storage(c.k_pool, "bf16"), block_table=c.block_table, seq_lens=c.seq_lens, Hkv=2, D=128, P=64)
    exact = oracle.summaries(**kw)
    rounded = oracle.summaries(summary_dtype="bf16", **kw)
    want = torch.from_numpy(exact).to(torch.bfloat16).to(torch.float64).numpy()   # fp64 -> bf16, one rounding
    np.testing.assert_array_equal(rounded, want)
    for b, n in enumerate(c.seq_lens):         # the rounding really happened on the real blocks
        nb = (int(n) + 63) // 64
        assert np.mean(rounded[b, :nb] != exact[b, :nb]) > 0.5   # short blocks often average to bf16 values


def test_bf16_summaries_change_nothing_when_means_are_bf16_values():
    """Every block holds one repeated bf16 key per group: its mean is already a bf16 value, so
    the bf16 mode gives the fp32 mode's scores, lists, outputs and lse exactly."""
    c = make_decode_case(B=2, Hq=8, Hkv=2, lens=[900, 300], top_k=3, dtype="bf16", seed=72)
    k = c.k_pool.copy()
    k[:] = k[:, :, :1, :]          # token 0 of each page repeated over the page
    c.k_pool = k
    kw = decode_inputs(c)
    a = oracle.decode(**kw)
    b = oracle.decode(summary_dtype="bf16", **kw)
    for key in ("scores", "idx", "o", "lse"):
        np.testing.assert_array_equal(a[key], b[key])


def test_bf16_summaries_scores_use_the_rounded_summaries():
    """Decode and prefill scores in the bf16 mode equal the fp32-mode scores computed from
    summaries that were rounded first (decode: through the precomputed-summary input)."""
    c = make_decode_case(B=2, Hq=8, Hkv=2, lens=[2000, 700], top_k=5, dtype="bf16", seed=73, permute=True)
    kw = decode_inputs(c)
    S = oracle.summaries(k_pool=kw["k_pool"], block_table=c.block_table, seq_lens=c.seq_lens, Hkv=2, D=128, P=64,
                         summary_dtype="bf16")
    a = oracle.decode(summary_dtype="bf16", **kw)
    b = oracle.decode(summaries_in=S, **kw)
    np.testing.assert_array_equal(a["scores"], b["scores"])
    np.testing.assert_array_equal(a["idx"], b["idx"])
    p = make_prefill_case(Hq=8, Hkv=2, past_len=640, T=200, top_k=3, dtype="bf16", seed=74)
    pk = prefill_inputs(p)
    r = oracle.prefill(summary_dtype="bf16", **pk)
    K = as_f64(storage(np.concatenate([logical_kv(p.k_pool, p.block_table, 0, 640), p.k_new]), "bf16"))
    q = as_f64(pk["q"])
    for tau in range(4):
        rows = slice(tau * 64, min(200, tau * 64 + 64))
        d = 10 + tau
        for g in range(2):
            qt = q[rows, g * 4:(g + 1) * 4].reshape(-1, 128).mean(axis=0)
            means = np.array([K[j * 64:(j + 1) * 64, g].mean(axis=0) for j in range(d)])
            Sb = torch.from_numpy(means).to(torch.bfloat16).to(torch.float64).numpy()
            np.testing.assert_allclose(r["scores"][tau, g, :d], Sb @ qt, rtol=1e-12, atol=1e-12)
