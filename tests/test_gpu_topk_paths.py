"""GPU parity of the top-k selection on crafted score rows, through msa_select.

The summary pool is written directly and every query head is the unit vector e_0, so block j of
group g scores exactly S[page_j][g][0]. Each row's kept list is compared with the oracle's top-k
of the same fp32 scores (as returned by the GPU): the same order applied to the same values, so
the lists must agree exactly. The distributions aim at the arithmetic of each selection path:
the group-maximum bound and its bin edge, survivors ranked 16 lanes each or one thread each, the
large-k select with its first pass on a score scale (and its fallback to key bins), the
memory-based select for rows beyond 16,384 blocks: heavy ties, ties at the top beyond the
survivor capacity, a spread narrower than the bins' float resolution, a huge dynamic range,
all-negative and subnormal scores, -inf from invalid page ids, forced blocks."""
import numpy as np
import pytest
import torch

import long_context_sparse_select_amd as msa
import oracle
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def crafted(kind, rng, shape):
    if kind == "normal":
        s = rng.standard_normal(shape)
    elif kind == "quantized":                       # a few dozen distinct values: ties everywhere
        s = np.round(rng.standard_normal(shape) * 4) / 4
    elif kind == "top_ties_600":                    # 600 blocks share the row maximum
        s = rng.standard_normal(shape)
        for r in np.ndindex(shape[:-1]):
            s[r][rng.choice(shape[-1], 600, replace=False)] = 10.0
    elif kind == "top_ties_3000":                   # more tied maxima than the survivor capacity
        s = rng.standard_normal(shape)
        for r in np.ndindex(shape[:-1]):
            s[r][rng.choice(shape[-1], 3000, replace=False)] = 10.0
    elif kind == "narrow":                          # spread ~1e-3 on 100: bins finer than an ulp
        s = 100.0 + 1e-3 * rng.standard_normal(shape)
    elif kind == "wide":                            # magnitudes from 1e-30 to 1e30, both signs
        s = np.sign(rng.standard_normal(shape)) * 10.0 ** rng.uniform(-30, 30, shape)
    elif kind == "negative":
        s = -1.0 - np.abs(rng.standard_normal(shape))
    elif kind == "subnormal":
        s = rng.standard_normal(shape) * 1e-40
    elif kind == "with_inf":                        # a few +inf and -inf among normal scores
        s = rng.standard_normal(shape)
        for r in np.ndindex(shape[:-1]):
            s[r][rng.choice(shape[-1], 3, replace=False)] = np.inf
            s[r][rng.choice(shape[-1], 40, replace=False)] = -np.inf
    elif kind == "offset":                          # spread 1e-2 on 1000: just under the value-bin guard
        s = 1000.0 + 1e-2 * rng.standard_normal(shape)
    elif kind == "quantized_fine":                  # steps of 1/64: a dozen ties per value near the k-th
        s = np.round(rng.standard_normal(shape) * 64) / 64
    elif kind.startswith("cluster_"):               # m distinct scores within 2e-4 (one value bin)
        _, where, m = kind.split("_")
        s = rng.standard_normal(shape)
        base = 5.0 if where == "top" else 1.72      # above every normal score, or ~700 normals above
        for r in np.ndindex(shape[:-1]):
            s[r][rng.choice(shape[-1], int(m), replace=False)] = base + 2e-4 * rng.random(int(m))
    elif kind == "outlier":                         # one huge score stretches the value range
        s = rng.standard_normal(shape)
        for r in np.ndindex(shape[:-1]):
            s[r][rng.integers(shape[-1])] = 1e6
    else:
        raise ValueError(kind)
    return s.astype(np.float32)


def run_case(kind, nbs, k, sink=0, local=0, bad=0, Hkv=2, G=4, seed=0):
    """nbs: blocks per sequence (full 64-token blocks, the last one 5 tokens short)."""
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
    if bad:                                          # invalid page ids inside the sequences
        for b, nb in enumerate(nbs):
            for j in rng.choice(nb, bad, replace=False):
                table[b, j] = -1 if j % 2 else num_pages + 7
    Hq = Hkv * G
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    q[:, :, 0] = 1.0
    dummy = torch.zeros(1, dtype=torch.bfloat16, device="cuda").expand(num_pages)   # K/V: not read
    cache = msa.KVCache(dummy, dummy, torch.from_numpy(S).cuda(), torch.from_numpy(table).cuda(),
                        torch.from_numpy(lens).cuda())
    cfg = msa.make_config(Hq, Hkv, k, dtype="bf16", keep_sink=sink)
    cfg.keep_local = local
    max_len = int(lens.max())
    idx = torch.empty((B, Hkv, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hkv, mb), dtype=torch.float32, device="cuda")
    msa.msa_select(cfg, q, cache, B, max_len, idx, scores_out=sc)
    torch.cuda.synchronize()
    got, gs = idx.cpu().numpy(), sc.cpu().numpy()
    for b, nb in enumerate(nbs):
        for g in range(Hkv):
            row = gs[b, g, :nb].astype(np.float64)
            ok = table[b, :nb] >= 0
            ok &= table[b, :nb] < num_pages
            expect_scores = np.where(ok, scores[b, g, :nb].astype(np.float64), -np.inf)
            # the score pass is exact here unless the GPU flushes subnormal products to zero
            if kind != "subnormal":
                np.testing.assert_array_equal(row, expect_scores, err_msg="scores b=%d g=%d" % (b, g))
            want = oracle.topk(row, k, sink, local)
            np.testing.assert_array_equal(got[b, g], want, err_msg="%s b=%d g=%d" % (kind, b, g))


CASES = [
    # (kind, blocks per sequence, k, keep_sink, keep_local, invalid page ids per sequence)
    ("normal", [16384, 9000], 64, 0, 0, 0),           # bound + survivors ranked 16 lanes each
    ("quantized", [16384, 5000], 64, 0, 0, 0),
    ("top_ties_600", [16384], 100, 0, 0, 0),          # 600 survivors: one thread per survivor
    ("top_ties_3000", [16384], 100, 0, 0, 0),         # beyond the survivor capacity: exact select
    ("narrow", [16384, 3000], 200, 1, 1, 0),
    ("normal", [16384, 12000], 1024, 0, 0, 0),        # large k: score-scale first pass
    ("quantized", [16384, 7000], 1024, 2, 2, 0),
    ("narrow", [16384], 1024, 0, 0, 0),
    ("wide", [16384, 2000], 3000, 0, 0, 0),
    ("negative", [16384], 700, 1, 0, 0),
    ("subnormal", [16384], 1024, 0, 0, 0),
    ("normal", [16384, 4000], 1024, 0, 0, 5),         # -inf scores: key-bin first pass
    ("normal", [16384], 4096, 0, 0, 0),
    # large k where the chosen value bin is crowded: finished in LDS up to 512 keys, refined by
    # key bins beyond (2000 distinct keys in one bin), ties inside a small bin
    ("cluster_top_2000", [16384, 9000], 1024, 0, 0, 0),
    ("cluster_mid_500", [16384, 12000], 1024, 0, 0, 0),
    ("cluster_mid_300", [16384], 900, 1, 1, 0),
    ("quantized_fine", [16384, 6000], 1024, 0, 0, 0),
    ("normal", [20000, 30000], 64, 0, 0, 0),          # memory-based select (rows > 16,384)
    ("quantized", [20000], 1024, 1, 1, 3),
    # small k on every distribution: the group-maximum bound on score-value bins, or key bins
    # where the value range is unusable (narrow against the magnitude, infinite, subnormal)
    ("narrow", [16384, 700], 64, 0, 0, 0),
    ("offset", [16384, 4100], 32, 0, 0, 0),
    ("wide", [16384, 4100], 64, 0, 0, 0),
    ("negative", [16384, 4100], 32, 0, 0, 0),
    ("subnormal", [16384, 4100], 64, 0, 0, 0),
    ("with_inf", [16384, 4100], 64, 0, 0, 0),
    ("outlier", [16384, 4100], 64, 0, 0, 0),
    ("quantized", [16384, 4100], 32, 1, 1, 4),
    ("normal", [4100, 16384], 200, 2, 0, 9),
]


@pytest.mark.parametrize("i", range(len(CASES)),
                         ids=["%s_n%d_k%d%s%s" % (c[0], c[1][0], c[2], "_forced" if c[3] or c[4] else "",
                                                  "_bad" if c[5] else "") for c in CASES])
def test_selection_paths_on_crafted_scores(i):
    kind, nbs, k, sink, local, bad = CASES[i]
    run_case(kind, nbs, k, sink, local, bad, seed=3100 + i)
