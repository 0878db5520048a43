"""GPU parity of the decode step's fused select-and-attend path (bf16, k <= 64, no forced blocks:
Step 1's TopK runs inside the attend launch, from the scores and chunk maxima of the scoring
launch) on crafted score rows, through msa_decode_step.

As in test_gpu_topk_paths, the summary pool is written directly and every query head is e_0, so
block j of group g scores exactly S[page_j][g][0]; the K/V pools are random, so the attend over
the kept blocks is real. Each row's list must equal the oracle's top-k of the GPU's own fp32
scores (the same order on the same values), and the outputs must equal the oracle's attention
over that list. The distributions aim at the selection's paths: the chunk-maximum bound on value
bins or key bins, rows with fewer chunks than k (every score a candidate), survivor chunks or
candidates beyond the LDS lists (the exact path), invalid page ids, and an appended token whose
block wins while its chunk's recorded maximum leaves it out."""
import numpy as np
import pytest
import torch

import long_context_sparse_select_amd as msa
import oracle
from gpu_util import assert_close, dev_tensor, host_f64, host_store, require_gpu
from test_gpu_topk_paths import crafted

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def build_case(kind, nbs, k, bad, seed, Hkv=2, G=4):
    rng = np.random.default_rng(seed)
    B = len(nbs)
    mb = max(nbs)
    num_pages = sum(nbs)
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((B, mb), -1, np.int32)
    off = 0
    for b, nb in enumerate(nbs):
        table[b, :nb] = perm[off:off + nb]
        off += nb
    lens = np.array([64 * nb - 5 for nb in nbs], np.int32)
    scores = crafted(kind, rng, (B, Hkv, mb))
    S = np.zeros((num_pages, Hkv, 128), np.float32)
    for b, nb in enumerate(nbs):
        S[table[b, :nb], :, 0] = scores[b, :, :nb].T
    if bad:
        for b, nb in enumerate(nbs):
            for j in rng.choice(nb, min(bad, nb), replace=False):
                table[b, j] = -1 if j % 2 else num_pages + 7
    Hq = Hkv * G
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    k_pool = torch.randn((num_pages, Hkv, 64, 128), generator=gen, device="cuda").to(torch.bfloat16)
    v_pool = torch.randn((num_pages, Hkv, 64, 128), generator=gen, device="cuda").to(torch.bfloat16)
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    q[:, :, 0] = 1.0
    cache = msa.KVCache(k_pool, v_pool, torch.from_numpy(S).cuda(), torch.from_numpy(table).cuda(),
                        torch.from_numpy(lens).cuda())
    cfg = msa.make_config(Hq, Hkv, k, dtype="bf16")
    return dict(B=B, Hq=Hq, Hkv=Hkv, mb=mb, k=k, num_pages=num_pages, table=table, lens=lens, scores=scores,
                q=q, cache=cache, cfg=cfg)


def run_and_check(c, k_new=None, v_new=None, expect_scores=True):
    B, Hq, Hkv, mb, k = c["B"], c["Hq"], c["Hkv"], c["mb"], c["k"]
    max_len = int(c["lens"].max())
    out = torch.empty_like(c["q"])
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    idx = torch.full((B, Hkv, k), -7, dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hkv, mb), dtype=torch.float32, device="cuda")
    msa.msa_decode_step(c["cfg"], c["q"], c["cache"], B, max_len, out, k_new=k_new, v_new=v_new, idx_out=idx,
                        scores_out=sc, lse_out=lse)
    torch.cuda.synchronize()
    got, gs = idx.cpu().numpy(), sc.cpu().numpy()
    table, num_pages = c["table"], c["num_pages"]
    for b in range(B):
        nb = (int(c["lens"][b]) + 63) // 64
        for g in range(Hkv):
            row = gs[b, g, :nb].astype(np.float64)
            if expect_scores:
                ok = (table[b, :nb] >= 0) & (table[b, :nb] < num_pages)
                want_s = np.where(ok, c["scores"][b, g, :nb].astype(np.float64), -np.inf)
                np.testing.assert_array_equal(row, want_s, err_msg="scores b=%d g=%d" % (b, g))
            np.testing.assert_array_equal(got[b, g], oracle.topk(row, k), err_msg="list b=%d g=%d" % (b, g))
    # outputs: the oracle's attention over the GPU's lists (blocks with an invalid page id hold no
    # tokens on either side: the GPU skips them, the oracle is handed -1 for them)
    idx_in = got.copy()
    for b in range(B):
        for g in range(Hkv):
            for e in range(k):
                j = idx_in[b, g, e]
                if j >= 0 and not (0 <= table[b, j] < num_pages):
                    idx_in[b, g, e] = -1
    cache = c["cache"]
    ref = oracle.decode(q=host_store(c["q"]), k_pool=host_store(cache.k_pages), v_pool=host_store(cache.v_pages),
                        block_table=table, seq_lens=c["lens"], Hq=Hq, Hkv=Hkv, top_k=k, scale=float(c["cfg"].softmax_scale),
                        summaries_in=np.zeros((B, mb, Hkv, 128)), idx_in=idx_in)
    assert_close(host_f64(out), ref["o"], "bf16", "o")
    assert_close(lse.cpu().numpy(), ref["lse"], "bf16", "lse", lse=True)
    return got, gs


CASES = [
    # (kind, blocks per sequence, k, invalid page ids per sequence)
    ("normal", [16384, 9000], 64, 0),          # the bound on value bins, ~k survivor chunks
    ("normal", [16384, 333], 1, 0),            # k = 1
    ("quantized", [16384, 5000], 64, 0),       # ties everywhere
    ("top_ties_600", [16384], 64, 0),          # ~600 chunks tie at the top: beyond the survivor list
    ("top_ties_3000", [16384, 8000], 48, 0),
    ("narrow", [16384, 700], 64, 0),           # key bins (range narrow against the magnitude)
    ("offset", [16384, 4100], 32, 0),
    ("wide", [9000, 4100], 64, 0),
    ("negative", [16384, 4100], 32, 0),
    ("subnormal", [4100, 2000], 64, 0),
    ("with_inf", [16384, 4100], 64, 0),        # +inf chunk maxima: key bins
    ("outlier", [16384, 4100], 64, 0),
    ("quantized", [16384, 4100], 32, 4),       # -inf scores of invalid page ids
    ("normal", [100, 30, 1023, 1025], 64, 0),  # fewer chunks than k: every score a candidate
    ("normal", [1, 2, 16, 17, 64], 64, 0),     # k >= blocks, tiny rows
    ("normal", [16384, 1000], 17, 9),
]


@pytest.mark.parametrize("i", range(len(CASES)),
                         ids=["%s_n%d_k%d%s" % (c[0], c[1][0], c[2], "_bad" if c[3] else "") for c in CASES])
def test_fused_select_on_crafted_scores(i):
    kind, nbs, k, bad = CASES[i]
    print("fused select: %s blocks %s k=%d bad=%d" % (kind, nbs, k, bad), flush=True)
    c = build_case(kind, nbs, k, bad, seed=5200 + i)
    # the score pass is exact here unless the GPU flushes subnormal products to zero
    run_and_check(c, expect_scores=kind != "subnormal")


@pytest.mark.parametrize("nbs", [[16384, 4000], [40, 16384]])
def test_fused_select_appended_block_wins(nbs):
    """A new token with key 1000 e_0: its block's recomputed summary scores far above every crafted
    score, though the chunk maximum the scoring launch records for that chunk leaves the block out;
    the block must be kept in every row."""
    c = build_case("normal", nbs, 64, 0, seed=5300 + len(nbs) + nbs[0])
    B, Hkv = c["B"], c["Hkv"]
    kn = torch.zeros((B, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    kn[:, :, 0] = 1000.0
    vn = torch.randn((B, Hkv, 128), device="cuda").to(torch.bfloat16)
    got, gs = run_and_check(c, k_new=kn, v_new=vn, expect_scores=False)
    for b in range(B):
        nb = (int(c["lens"][b]) + 63) // 64
        for g in range(Hkv):
            assert nb - 1 in got[b, g], (b, g)
            assert gs[b, g, nb - 1] == gs[b, g, :nb].max()
