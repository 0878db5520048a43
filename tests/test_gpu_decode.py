"""GPU parity of the decode path (block summaries, Step 1 select, Step 2 attend, decode step)
against the CPU oracle, through the C ABI. Sizes span several workgroup tiles with ragged tails;
full-size workloads are checked end to end (the 1M-token case entirely, the mixed batch on
sampled sequences)."""
import numpy as np
import pytest
import torch

import long_context_sparse_select_amd as msa
import oracle
from synth import make_decode_case, make_decode_case_torch, workload, storage, round_to_bf16
from gpu_util import (Dev, assert_close, check_index_sets, check_scores, dev_tensor, full_decode_check,
                      host_f64, host_store, index_query_abs_bound, oracle_inputs, require_gpu, run_decode,
                      to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


SMALL = [
    # (name, kwargs)
    ("fp32_g8_4k", dict(B=1, Hq=8, Hkv=1, lens=[4096], top_k=16, dtype="f32", plant=("count", 3))),
    ("bf16_g4_ragged", dict(B=3, Hq=32, Hkv=8, lens=[8192, 5000, 131], top_k=32, dtype="bf16",
                            plant=("frac", 0.01), permute=True)),
    ("bf16_diagram_g3", dict(B=2, Hq=6, Hkv=2, lens=[1000, 64], top_k=4, dtype="bf16")),
    ("f32_g2_tail", dict(B=2, Hq=4, Hkv=2, lens=[2049, 63], top_k=5, dtype="f32", permute=True)),
    ("bf16_g1", dict(B=1, Hq=4, Hkv=4, lens=[3333], top_k=7, dtype="bf16")),
    ("bf16_g8_bigk", dict(B=1, Hq=16, Hkv=2, lens=[20000], top_k=300, dtype="bf16")),
    # enough (sequence, group) rows that the attend runs four blocks per workgroup; short rows
    # leave chunks with 1..3 attended blocks
    ("bf16_g2_wide", dict(B=6, Hq=16, Hkv=8, lens=[70000, 4096, 65, 1, 33333, 9000], top_k=64,
                          dtype="bf16", permute=True)),
    # large k: the exact selection path (range-refined threshold + ordered compaction)
    ("bf16_g4_k1024", dict(B=1, Hq=8, Hkv=2, lens=[262144], top_k=1024, dtype="bf16", permute=True)),
    ("f32_g2_k700_ragged", dict(B=2, Hq=4, Hkv=2, lens=[100000, 45000], top_k=700, dtype="f32")),
    # one (sequence, group) row with k above 512 (the fp32 workload's head layout): the attend must
    # still fit its splits in one merge workgroup (at most 256), so every list entry is attended
    ("bf16_g8_hkv1_k1024", dict(B=1, Hq=8, Hkv=1, lens=[70001], top_k=1024, dtype="bf16", permute=True)),
    ("f32_g8_hkv1_k600", dict(B=1, Hq=8, Hkv=1, lens=[40000], top_k=600, dtype="f32")),
    # 160 (sequence, group) rows: sixteen blocks per workgroup (four chunks of four), ragged rows
    ("bf16_g4_b20_many_rows", dict(B=20, Hq=32, Hkv=8, lens=[20000, 1, 4100, 64, 65, 127, 8191, 5000, 12345, 300,
                                                             16384, 2, 999, 4096, 7777, 640, 641, 19999, 3000, 10],
                                   top_k=64, dtype="bf16", permute=True)),
    # 256 (sequence, group) rows: one workgroup per row attends the whole list and writes the final
    # output (no split, no merge launch); ragged and tiny rows
    ("bf16_g4_b32_single_split", dict(B=32, Hq=32, Hkv=8, lens=[1, 63, 64, 65] + [97 * i + 5 for i in range(1, 29)],
                                      top_k=16, dtype="bf16", permute=True)),
    ("f32_g2_b64_single_split", dict(B=64, Hq=8, Hkv=4, lens=[17 * i + 3 for i in range(64)], top_k=6, dtype="f32")),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_build_summaries(name, kw):
    c = make_decode_case(seed=21, **kw)
    d = to_device(c)
    torch.cuda.synchronize()
    inputs = oracle_inputs(d)
    S64 = oracle.summaries(k_pool=inputs["k_pool"], block_table=c.block_table, seq_lens=c.seq_lens,
                           Hkv=c.Hkv, D=c.D, P=c.P)
    S = d.S.cpu().numpy()
    for b in range(c.B):
        nb = (int(c.seq_lens[b]) + 63) // 64
        got = S[c.block_table[b, :nb]]                    # [nb][Hkv][D]
        np.testing.assert_allclose(got, S64[b, :nb], rtol=1e-5, atol=2e-6)


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_select(name, kw):
    c = make_decode_case(seed=22, **kw)
    d = to_device(c)
    mb = (c.max_seq_len + 63) // 64
    idx = torch.empty((c.B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
    scores = torch.full((c.B, c.Hkv, mb), float("nan"), dtype=torch.float32, device="cuda")
    msa.msa_select(d.cfg, d.q, d.cache, c.B, c.max_seq_len, idx, scores_out=scores)
    torch.cuda.synchronize()
    inputs = oracle_inputs(d)
    ref = oracle.decode(**inputs)
    S64 = oracle.summaries(k_pool=inputs["k_pool"], block_table=c.block_table, seq_lens=c.seq_lens,
                           Hkv=c.Hkv, D=c.D, P=c.P)
    nb = (c.seq_lens.astype(np.int64) + 63) // 64
    bound = index_query_abs_bound(host_f64(d.q), S64, c.Hkv)
    gs = scores.cpu().numpy()
    check_scores(gs, ref["scores"], bound, nb)
    check_index_sets(idx.cpu().numpy(), gs, ref["scores"], bound, nb, c.top_k)


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_attend_with_oracle_indices(name, kw):
    """Stage 2 alone: the GPU attends over the oracle's own index lists."""
    c = make_decode_case(seed=23, **kw)
    d = to_device(c)
    inputs = oracle_inputs(d)
    ref = oracle.decode(**inputs)
    idx = torch.from_numpy(ref["idx"]).cuda()
    out = torch.empty_like(d.q)
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    msa.msa_attend(d.cfg, d.q, d.cache, c.B, c.max_seq_len, idx, out, lse_out=lse)
    torch.cuda.synchronize()
    assert_close(host_f64(out), ref["o"], c.dtype, "o")
    assert_close(lse.cpu().numpy(), ref["lse"], c.dtype, "lse", lse=True)


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_decode_step(name, kw):
    c = make_decode_case(seed=24, **kw)
    d = to_device(c)
    res = run_decode(d)
    full_decode_check(d, res)


def test_decode_step_appends_token():
    """k_new/v_new land at position len-1 and that block's summary is recomputed."""
    c = make_decode_case(B=3, Hq=32, Hkv=8, lens=[777, 64, 4097], top_k=8, dtype="bf16", seed=25, permute=True)
    d = to_device(c)
    r = np.random.default_rng(5)
    kn = round_to_bf16(r.standard_normal((c.B, c.Hkv, c.D), dtype=np.float32) * 3)
    vn = round_to_bf16(r.standard_normal((c.B, c.Hkv, c.D), dtype=np.float32))
    res = run_decode(d, k_new=dev_tensor(storage(kn, "bf16")), v_new=dev_tensor(storage(vn, "bf16")))
    # the host copy of the cache with the same token written
    k2, v2 = c.k_pool.copy(), c.v_pool.copy()
    for b in range(c.B):
        t = int(c.seq_lens[b]) - 1
        k2[c.block_table[b, t // 64], :, t % 64] = kn[b]
        v2[c.block_table[b, t // 64], :, t % 64] = vn[b]
    np.testing.assert_array_equal(host_store(d.k), storage(k2, "bf16"))
    np.testing.assert_array_equal(host_store(d.v), storage(v2, "bf16"))
    S64 = oracle.summaries(k_pool=storage(k2, "bf16"), block_table=c.block_table, seq_lens=c.seq_lens,
                           Hkv=c.Hkv, D=c.D, P=c.P)
    S = d.S.cpu().numpy()
    for b in range(c.B):
        nb = (int(c.seq_lens[b]) + 63) // 64
        np.testing.assert_allclose(S[c.block_table[b, :nb]], S64[b, :nb], rtol=1e-5, atol=2e-6)
    full_decode_check(d, res, S64=S64)


def test_empty_and_tiny_sequences():
    c = make_decode_case(B=4, Hq=8, Hkv=2, lens=[0, 1, 64, 65], top_k=3, dtype="bf16", seed=26)
    d = to_device(c)
    res = run_decode(d)
    o = host_f64(res["o"])
    assert np.all(o[0] == 0) and np.all(np.isneginf(res["lse"].cpu().numpy()[0]))
    assert np.all(res["idx"].cpu().numpy()[0] == -1)
    full_decode_check(d, res)


def test_invalid_page_ids_are_never_read():
    c = make_decode_case(B=2, Hq=8, Hkv=2, lens=[1000, 1000], top_k=4, dtype="bf16", seed=27)
    d = to_device(c)
    torch.cuda.synchronize()
    bad = c.block_table.copy()
    bad[0, 3] = c.num_pages + 1000     # out of range
    bad[0, 5] = -7
    d.table.copy_(torch.from_numpy(bad))
    res = run_decode(d)
    s = res["scores"].cpu().numpy()
    assert np.isneginf(s[0, :, 3]).all() and np.isneginf(s[0, :, 5]).all()
    idx = res["idx"].cpu().numpy()
    assert not np.isin(idx[0], [3, 5]).any()
    # sequence 1 is untouched by sequence 0's bad entries
    d.table.copy_(torch.from_numpy(c.block_table))
    res2 = run_decode(d)
    np.testing.assert_array_equal(host_store(res["o"])[1], host_store(res2["o"])[1])


def test_determinism_and_page_permutation():
    c = make_decode_case(B=2, Hq=32, Hkv=8, lens=[9000, 3000], top_k=16, dtype="bf16", seed=28)
    d = to_device(c)
    r1 = run_decode(d)
    r2 = run_decode(d)
    for key in ("o", "lse", "idx", "scores"):
        assert torch.equal(r1[key], r2[key]), key
    perm = np.random.default_rng(1).permutation(c.num_pages)
    k2 = torch.empty_like(d.k); k2[torch.from_numpy(perm).cuda()] = d.k
    v2 = torch.empty_like(d.v); v2[torch.from_numpy(perm).cuda()] = d.v
    t2 = np.where(c.block_table >= 0, perm[np.maximum(c.block_table, 0)], -1).astype(np.int32)
    c2 = make_decode_case(B=2, Hq=32, Hkv=8, lens=[9000, 3000], top_k=16, dtype="bf16", seed=28)
    c2.block_table = t2
    d2 = to_device(c2, build=False)
    d2.k.copy_(k2); d2.v.copy_(v2)
    msa.msa_build_summaries(d2.cfg, d2.cache, c2.B, c2.max_seq_len)
    r3 = run_decode(d2)
    for key in ("o", "lse", "idx", "scores"):
        assert torch.equal(r1[key], r3[key]), key


def test_metamorphic_scaling_and_constant_values():
    c = make_decode_case(B=2, Hq=32, Hkv=8, lens=[5000, 7000], top_k=16, dtype="bf16", seed=29)
    d = to_device(c)
    r1 = run_decode(d)
    d.q.mul_(2.0)                         # exact in bf16
    r2 = run_decode(d)
    assert torch.equal(r2["scores"], r1["scores"] * 2)
    assert torch.equal(r2["idx"], r1["idx"])
    d.v.fill_(1.0)
    r3 = run_decode(d)
    assert torch.all(r3["o"].float() == 1.0)


def test_weights_sum_to_one():
    """With the oracle's logits, sum_t exp(z_t - lse_gpu) = 1 over the attended tokens."""
    c = make_decode_case(B=1, Hq=8, Hkv=2, lens=[3000], top_k=6, dtype="f32", seed=30)
    d = to_device(c)
    res = run_decode(d)
    idx = res["idx"].cpu().numpy()
    lse = res["lse"].cpu().numpy()
    K = c.k_pool
    for h in range(8):
        g = h // 4
        toks = np.concatenate([np.arange(j * 64, min(3000, j * 64 + 64)) for j in idx[0, g] if j >= 0])
        rows = K[c.block_table[0, toks // 64], g, toks % 64].astype(np.float64)
        z = c.scale * rows @ c.q[0, h].astype(np.float64)
        assert abs(np.exp(z - lse[0, h]).sum() - 1.0) < 1e-5


def test_batch_subset_independence():
    lens = [7000, 300, 12000]
    c = make_decode_case(B=3, Hq=32, Hkv=8, lens=lens, top_k=16, dtype="bf16", seed=31, permute=True)
    d = to_device(c)
    full = run_decode(d)
    for b in range(3):
        sub = make_decode_case(B=3, Hq=32, Hkv=8, lens=lens, top_k=16, dtype="bf16", seed=31, permute=True)
        sub.B = 1
        sub.q = c.q[b:b + 1]
        sub.block_table = c.block_table[b:b + 1]
        sub.seq_lens = c.seq_lens[b:b + 1]
        ds = to_device(sub)
        one = run_decode(ds, max_len=int(c.seq_lens.max()))
        assert torch.equal(one["idx"][0], full["idx"][b])
        assert torch.equal(one["scores"][0], full["scores"][b])
        assert_close(host_f64(one["o"][0]), host_f64(full["o"][b]), "bf16", "o")


# ----------------------------------------------------------------------------- full size
def test_full_fp32_4k():
    c = make_decode_case(**workload("decode_f32_4k", seed=0))
    d = to_device(c)
    full_decode_check(d, run_decode(d))


@pytest.mark.parametrize("name", ["decode_bf16_1m_paged", "decode_bf16_b8_128k"])
def test_full_size_decode(name):
    kw = workload(name, seed=0)
    c = make_decode_case_torch(**kw)
    d = to_device(c)
    res = run_decode(d)
    off = full_decode_check(d, res)
    print("%s: %d rows differ from the oracle inside the band" % (name, off))
    # planted blocks are found (input-recipe sanity, not parity)
    idx = res["idx"].cpu().numpy()
    hit = sum(len(set(v) & set(idx[b, g])) for (b, g), v in c.planted.items())
    tot = sum(len(v) for v in c.planted.values())
    assert hit / tot > 0.8


def test_full_size_decode_large_k():
    """The pages' operating point: 1M tokens, k = 1024 of 16,384 blocks (about 6 %)."""
    kw = dict(workload("decode_bf16_1m_paged", seed=0), top_k=1024)
    c = make_decode_case_torch(**kw)
    d = to_device(c)
    res = run_decode(d)
    off = full_decode_check(d, res)
    print("1M k=1024: %d rows differ from the oracle inside the band" % off)


@pytest.mark.parametrize("B,n,k,sink,local", [(1, 1 << 20, 65, 0, 0), (1, 1 << 20, 256, 0, 0),
                                              (2, 1 << 19, 128, 1, 1), (1, 1 << 18, 256, 0, 0),
                                              (1, 1 << 18, 192, 1, 1), (2, 1 << 17, 128, 0, 0)])
def test_full_size_decode_fused_large_k(B, n, k, sink, local):
    """k from 65 to 256 on rows of at least 2k runs of 8 blocks (down to exactly 2k at 256k
    tokens, k = 256): Step 1's top-k runs inside the attend launch (run-maximum bound, ~k .. 2k
    candidates ranked), with and without forced blocks; the lists and outputs against the
    oracle."""
    kw = dict(workload("decode_bf16_1m_paged", seed=0), B=B, lens=[n] * B, top_k=k)
    c = make_decode_case_torch(**kw)
    d = to_device(c)
    d.cfg.keep_sink, d.cfg.keep_local = sink, local
    res = run_decode(d)
    off = full_decode_check(d, res)
    print("B=%d n=%d k=%d: %d rows differ from the oracle inside the band" % (B, n, k, off))


@pytest.mark.parametrize("k", [300, 1500])
def test_large_k_all_scores_tied(k):
    """Every block scores exactly 0 (all keys zero): the kept blocks are the k smallest indices."""
    c = make_decode_case(B=2, Hq=8, Hkv=2, lens=[130000, 64 * 2000 - 5], top_k=k, dtype="bf16", seed=41,
                         permute=True)
    d = to_device(c, build=False)
    d.k.zero_()
    msa.msa_build_summaries(d.cfg, d.cache, c.B, c.max_seq_len)
    idx = torch.empty((c.B, c.Hkv, k), dtype=torch.int32, device="cuda")
    msa.msa_select(d.cfg, d.q, d.cache, c.B, c.max_seq_len, idx)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for b in range(c.B):
        nb = (int(c.seq_lens[b]) + 63) // 64
        want = np.arange(min(k, nb), dtype=np.int32)
        for g in range(c.Hkv):
            assert np.array_equal(got[b, g, :len(want)], want), (b, g)
            assert np.all(got[b, g, len(want):] == -1)


@pytest.fixture(scope="module")
def mixed_run():
    """The batch-32 mixed-length workload, one decode step on the GPU."""
    require_gpu()
    kw = workload("decode_bf16_mixed_b32", seed=0)
    c = make_decode_case_torch(**kw)
    d = to_device(c)
    return c, d, run_decode(d)


# ranks in ascending length order: the shortest, the longest and six between
@pytest.mark.parametrize("ranks", [(0, 4, 9, 13), (18, 22, 27, 31)])
def test_full_size_mixed_batch(mixed_run, ranks):
    c, d, res = mixed_run
    lens = c.seq_lens
    order = np.argsort(lens, kind="stable")
    for b in (int(order[r]) for r in ranks):
        print("mixed batch: sequence %d, %d tokens" % (b, int(lens[b])), flush=True)
        nb = (int(lens[b]) + 63) // 64
        pages = torch.from_numpy(c.block_table[b, :nb].astype(np.int64)).cuda()
        sub_k = host_store(d.k.index_select(0, pages))
        sub_v = host_store(d.v.index_select(0, pages))
        inputs = dict(q=host_store(d.q[b:b + 1]), k_pool=sub_k, v_pool=sub_v,
                      block_table=np.arange(nb, dtype=np.int32)[None], seq_lens=lens[b:b + 1],
                      Hq=c.Hq, Hkv=c.Hkv, top_k=c.top_k, scale=c.scale, P=c.P)
        ref = oracle.decode(**inputs)
        S64 = oracle.summaries(k_pool=sub_k, block_table=inputs["block_table"], seq_lens=lens[b:b + 1],
                               Hkv=c.Hkv, D=c.D, P=c.P)
        bound = index_query_abs_bound(host_f64(d.q[b:b + 1]), S64, c.Hkv)
        gs = res["scores"][b:b + 1, :, :nb].cpu().numpy()
        check_scores(gs, ref["scores"], bound, np.array([nb]))
        gi = res["idx"][b:b + 1].cpu().numpy()
        same = check_index_sets(gi, gs, ref["scores"], bound, np.array([nb]), c.top_k)
        if not same.all():
            ref = oracle.decode(idx_in=gi, **inputs)
        assert_close(host_f64(res["o"][b:b + 1]), ref["o"], "bf16", "o b=%d" % b)
        assert_close(res["lse"][b:b + 1].cpu().numpy(), ref["lse"], "bf16", "lse b=%d" % b, lse=True)


def test_score_entry_point_matches_select_scores():
    """msa_score (scoring alone) writes exactly the scores msa_select reports."""
    c = make_decode_case(B=3, Hq=32, Hkv=8, lens=[9000, 130, 4096], top_k=8, dtype="bf16", seed=32, permute=True)
    d = to_device(c)
    mb = (c.max_seq_len + 63) // 64
    s1 = torch.full((c.B, c.Hkv, mb), float("nan"), dtype=torch.float32, device="cuda")
    s2 = torch.full_like(s1, float("nan"))
    idx = torch.empty((c.B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
    msa.msa_score(d.cfg, d.q, d.cache, c.B, c.max_seq_len, s1)
    msa.msa_select(d.cfg, d.q, d.cache, c.B, c.max_seq_len, idx, scores_out=s2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)


@pytest.mark.parametrize("Hkv,lens", [
    (4, [300 * 64, 300 * 64 - 5, 285 * 64, 290 * 64 - 3, 272 * 64, 256 * 64, 100 * 64 + 7, 64, 1]),
    (8, [2100 * 64, 64, 1000 * 64 + 3, 1800 * 64]),
    (8, [17000 * 64, 64, 9000 * 64 - 1]),
])
def test_score_tails_past_each_end(Hkv, lens):
    """msa_score writes -inf over every block past each sequence's end and leaves nothing else
    unwritten, into a buffer that starts as NaN: tails of no block, inside the last scoring
    chunk, one chunk past the end, several, and a 544 KB tail that several chunks past the end
    split between them (one writer per 256 KB)."""
    gen = make_decode_case_torch if max(lens) > 1 << 18 else make_decode_case
    c = gen(B=len(lens), Hq=2 * Hkv, Hkv=Hkv, lens=lens, top_k=8, dtype="bf16", seed=41, permute=True)
    d = to_device(c)
    mb = (c.max_seq_len + 63) // 64
    s1 = torch.full((c.B, c.Hkv, mb), float("nan"), dtype=torch.float32, device="cuda")
    msa.msa_score(d.cfg, d.q, d.cache, c.B, c.max_seq_len, s1)
    torch.cuda.synchronize()
    s = s1.cpu().numpy()
    for b, n in enumerate(lens):
        nb = (n + 63) // 64
        assert np.all(np.isfinite(s[b, :, :nb])), "b=%d: a block before the end is not scored" % b
        assert np.all(np.isneginf(s[b, :, nb:])), "b=%d: %d entries past the end not -inf" % (
            b, int(np.sum(~np.isneginf(s[b, :, nb:]))))
    s2 = torch.full_like(s1, float("nan"))
    idx = torch.empty((c.B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
    msa.msa_select(d.cfg, d.q, d.cache, c.B, c.max_seq_len, idx, scores_out=s2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)


EDGE = [
    # the largest top-k the library accepts (4096 of 5000 blocks: 256 splits, the widest merge)
    ("bf16_k4096_max", dict(B=1, Hq=8, Hkv=2, lens=[64 * 5000 - 17], top_k=4096, dtype="bf16", permute=True)),
    # the most KV heads (64, G = 1) and the smallest k
    ("bf16_hkv64_k1", dict(B=2, Hq=64, Hkv=64, lens=[3000, 64], top_k=1, dtype="bf16", permute=True)),
    # the largest group (G = 8) in fp32 with k = 1
    ("f32_g8_k1", dict(B=2, Hq=16, Hkv=2, lens=[777, 5000], top_k=1, dtype="f32")),
]


@pytest.mark.parametrize("name,kw", EDGE, ids=[e[0] for e in EDGE])
def test_decode_step_edge_sizes(name, kw):
    c = make_decode_case(seed=27, **kw)
    d = to_device(c)
    full_decode_check(d, run_decode(d))


def test_graph_replays_match_eager_calls():
    """The decode step captured in a HIP graph (as the benchmark times it) gives, on every replay
    with eager work and synchronisations in between, exactly the eager call's outputs."""
    c = make_decode_case(B=2, Hq=32, Hkv=8, lens=[20000, 3000], top_k=32, dtype="bf16", seed=28, permute=True)
    d = to_device(c)
    mb = (c.max_seq_len + 63) // 64
    out = torch.empty_like(d.q)
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    idx = torch.empty((c.B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(msa.msa_workspace_size(d.cfg, msa.MSA_OP_DECODE, c.B, c.max_seq_len), dtype=torch.uint8,
                     device="cuda")

    def step():
        msa.msa_decode_step(d.cfg, d.q, d.cache, c.B, c.max_seq_len, out, idx_out=idx, lse_out=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    want = (out.clone(), lse.clone(), idx.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        out.zero_(); lse.zero_(); idx.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want[0]) and torch.equal(lse, want[1]) and torch.equal(idx, want[2]), r
        step()            # eager work between replays
        torch.cuda.synchronize()


def test_full_size_decode_1m_with_append():
    """The benchmark's timed configuration: the 1M-token step with the new token's K/V appended
    (its block's summary and score recomputed in the scoring launch), checked end to end against
    the oracle run on the cache after the append."""
    kw = workload("decode_bf16_1m_paged", seed=0)
    c = make_decode_case_torch(**kw)
    d = to_device(c)
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    kn = torch.randn((c.B, c.Hkv, c.D), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((c.B, c.Hkv, c.D), generator=g, device="cuda").to(torch.bfloat16)
    res = run_decode(d, k_new=kn, v_new=vn)
    full_decode_check(d, res)
    t = int(c.seq_lens[0]) - 1
    page = int(c.block_table[0, t // 64])
    assert torch.equal(d.k[page, :, t % 64], kn[0]) and torch.equal(d.v[page, :, t % 64], vn[0])


@pytest.mark.parametrize("entry", ["decode_step", "attend"])
def test_bf16_p_rounding_bound(entry):
    """The bf16 attend kernels weight V by P rounded to bf16 (relative error <= 2^-8, round to
    nearest) while the softmax denominator sums the fp32 P; with the bf16 rounding of the output the
    error is bounded per element by 2^-8 (sum_t w_t |v_t| + |o|) + 1e-6 (w: the oracle's exact
    weights). Near-flat logits (a small query) spread the weight over every token, and V is distinct
    per token with a large common offset, which is where a mismatch of numerator and denominator
    weights shows most. k covers every block, so the oracle's weight list is in token order."""
    c = make_decode_case(B=2, Hq=8, Hkv=2, lens=[700, 2000], top_k=40, dtype="bf16", seed=61)
    r = np.random.default_rng(61)
    c.q = (0.05 * r.standard_normal(c.q.shape)).astype(np.float32)
    nb_pages = c.v_pool.shape[0]
    t_index = np.arange(64, dtype=np.float32)[None, None, :, None]
    c.v_pool = (3.0 + 0.01 * (t_index + 64 * np.arange(nb_pages, dtype=np.float32)[:, None, None, None] % 97)
                + 0.1 * r.standard_normal(c.v_pool.shape)).astype(np.float32)
    d = to_device(c)
    if entry == "decode_step":
        res = run_decode(d)
        out, lse = res["o"], res["lse"]
    else:
        idx = torch.from_numpy(np.tile(np.arange(40, dtype=np.int32), (c.B, c.Hkv, 1))).cuda()
        out = torch.empty_like(d.q)
        lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
        msa.msa_attend(d.cfg, d.q, d.cache, c.B, c.max_seq_len, idx, out, lse_out=lse)
        torch.cuda.synchronize()
    inputs = oracle_inputs(d)
    ref = oracle.decode(want_weights=True, **inputs)
    v64 = host_f64(d.v)
    G = c.Hq // c.Hkv
    got = host_f64(out)
    for b in range(c.B):
        N = int(c.seq_lens[b])
        assert list(ref["idx"][b, 0][:(N + 63) // 64]) == list(range((N + 63) // 64))
        t = np.arange(N)
        for h in range(c.Hq):
            g = h // G
            vt = v64[c.block_table[b, t // 64], g, t % 64, :]        # [N][D] in token order
            w = ref["w"][b, h, :N]
            assert abs(w.sum() - 1.0) < 1e-12
            bound = 2.0 ** -8 * (w @ np.abs(vt) + np.abs(ref["o"][b, h])) + 1e-6
            err = np.abs(got[b, h] - ref["o"][b, h])
            assert np.all(err <= bound), (entry, b, h, float((err / bound).max()))
    assert_close(lse.cpu().numpy(), ref["lse"], "bf16", "lse", lse=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_outputs_do_not_depend_on_workspace_contents(dtype):
    """Workspace scores are written only up to each sequence's length (the top-k and the fused
    selection read no further), so a workspace full of NaN bytes must give the same step and the
    same selection as a zeroed one. Mixed lengths, so most chunks of the short rows are skipped;
    bf16 takes the fused select-and-attend path, f32 the separate top-k."""
    c = make_decode_case(B=4, Hq=8, Hkv=2, lens=[100, 3000, 64 * 700 - 3, 9000], top_k=8, dtype=dtype, seed=81)
    d = to_device(c)
    B, max_len = c.B, c.max_seq_len
    n = msa.msa_workspace_size(d.cfg, msa.MSA_OP_DECODE, B, max_len)
    results = []
    for fill in (0x00, 0xFF):
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(d.q)
        lse = torch.empty((B, c.Hq), dtype=torch.float32, device="cuda")
        idx = torch.empty((B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
        msa.msa_decode_step(d.cfg, d.q, d.cache, B, max_len, out, idx_out=idx, lse_out=lse, workspace=ws)
        sel = torch.empty_like(idx)
        ws.fill_(fill)
        msa.msa_select(d.cfg, d.q, d.cache, B, max_len, sel, workspace=ws)
        torch.cuda.synchronize()
        results.append((out, lse, idx, sel))
    for name, x, y in zip(("o", "lse", "idx", "select"), results[0], results[1]):
        assert torch.equal(x, y), name
    assert torch.equal(results[0][2], results[0][3])
