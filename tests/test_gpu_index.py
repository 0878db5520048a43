"""GPU parity of the index branch of Step 1 (single-head index keys, token scores, Block Max Pool,
TopK) against the CPU oracle, through the C ABI.

Tolerance: a block score is a max over tokens of fp32 dot products, so it is within
1e-5 * max(|ref|, m_j) of the fp64 score, m_j = max over the block's valid tokens of
sum_d |q_idx,d * K_idx,t,d| (the summand scale of the token that may win). Index sets follow the
same rule as the mean-key select: bit-exact against the oracle's top-k of the GPU's own fp32
scores, and the band rule against the fp64 scores.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_select_amd as msa
import oracle
from synth import make_index_case, make_index_case_torch, storage
from gpu_util import SCORE_RTOL, check_index_sets, dev_tensor, host_store, require_gpu
from helpers import as_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


SMALL = [
    ("bf16_g8_ragged_perm", dict(B=3, Hkv=8, lens=[8192, 5000, 131], top_k=32, dtype="bf16", permute=True)),
    ("f32_g1_tail", dict(B=2, Hkv=1, lens=[2049, 63], top_k=5, dtype="f32", permute=True)),
    ("bf16_g2_k_over_nb", dict(B=2, Hkv=2, lens=[1000, 64], top_k=40, dtype="bf16")),
    ("f32_g8_many_rows", dict(B=5, Hkv=8, lens=[20000, 1, 65, 4097, 640], top_k=16, dtype="f32", permute=True)),
    # large k: the exact range-refined selection
    ("bf16_g4_k1024", dict(B=1, Hkv=4, lens=[262144], top_k=1024, dtype="bf16", permute=True,
                           plant=("frac", 0.01))),
    # wide groups: index queries staged in several passes (bf16 32 groups, fp32 64 groups)
    ("bf16_g32", dict(B=2, Hkv=32, lens=[5000, 130], top_k=8, dtype="bf16")),
    ("f32_g64", dict(B=1, Hkv=64, lens=[3000], top_k=4, dtype="f32")),
    # 64-dim index keys
    ("bf16_di64_ragged", dict(B=3, Hkv=8, lens=[9000, 130, 4097], top_k=16, dtype="bf16", permute=True, Di=64)),
    ("f32_di64_g4", dict(B=2, Hkv=4, lens=[5000, 64], top_k=8, dtype="f32", Di=64)),
]


def device_case(c):
    qi = c.q_idx if isinstance(c.q_idx, torch.Tensor) else dev_tensor(storage(c.q_idx, c.dtype))
    ik = c.index_keys if isinstance(c.index_keys, torch.Tensor) else dev_tensor(storage(c.index_keys, c.dtype))
    table = torch.from_numpy(np.ascontiguousarray(c.block_table)).cuda()
    lens = torch.from_numpy(np.ascontiguousarray(c.seq_lens)).cuda()
    cfg = msa.make_config(c.Hkv, c.Hkv, c.top_k, dtype=c.dtype)
    return cfg, qi, ik, table, lens


def run_index(c, max_len=None, table=None, scores=True):
    cfg, qi, ik, tab, lens = device_case(c)
    if table is not None:
        tab = torch.from_numpy(np.ascontiguousarray(table)).cuda()
    max_len = c.max_seq_len if max_len is None else max_len
    mb = (max_len + 63) // 64
    idx = torch.empty((c.B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
    sc = (torch.full((c.B, c.Hkv, max(mb, 1)), float("nan"), dtype=torch.float32, device="cuda")
          if scores else None)
    msa.msa_select_index(cfg, qi, ik, tab, lens, c.B, max_len, idx, scores_out=sc)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (sc.cpu().numpy()[:, :, :mb] if scores else None), host_store(qi), host_store(ik)


def token_abs_bound(q_store, k_store, table, lens, num_pages):
    """m[b][g][j] = max over block j's valid tokens of sum_d |q_idx[b][g][d] * K_idx[t][d]| (0 for a
    bad page or an empty block)."""
    q = np.abs(as_f64(q_store))
    k = np.abs(as_f64(k_store))
    B, Hkv, _ = q.shape
    out = np.zeros((B, Hkv, table.shape[1]))
    for b in range(B):
        N = int(lens[b])
        for j in range((N + 63) // 64):
            p = int(table[b, j])
            if 0 <= p < num_pages:
                n = min(64, N - 64 * j)
                out[b, :, j] = (k[p, :n] @ q[b].T).max(axis=0)
    return out


def check_index_scores(gs, ref, bound, nb):
    """Same -inf pattern on the candidate blocks, -inf past them, finite scores within the bound."""
    for b in range(ref.shape[0]):
        n = int(nb[b])
        g_s, r_s = gs[b, :, :n].astype(np.float64), ref[b, :, :n]
        assert np.array_equal(np.isneginf(g_s), np.isneginf(r_s)), "-inf pattern differs (b=%d)" % b
        fin = np.isfinite(r_s)
        tol = SCORE_RTOL * np.maximum(np.abs(r_s[fin]), bound[b, :, :n][fin])
        err = np.abs(g_s[fin] - r_s[fin])
        assert np.all(err <= tol), "score mismatch b=%d worst err/tol %g" % (b, float((err / tol).max()))
        assert np.all(np.isneginf(gs[b, :, n:]))


def full_check(c, gi, gs, qs, ks, table=None, keep_sink=0, keep_local=0):
    table = c.block_table if table is None else table
    ref = oracle.select_index(q_idx=qs, index_keys=ks, block_table=table, seq_lens=c.seq_lens, top_k=c.top_k,
                              keep_sink=keep_sink, keep_local=keep_local)
    mb = gs.shape[2]
    nb = (c.seq_lens.astype(np.int64) + 63) // 64
    bound = token_abs_bound(qs, ks, table, c.seq_lens, c.num_pages)
    check_index_scores(gs, ref["scores"][:, :, :mb], bound[:, :, :mb], nb)
    same = check_index_sets(gi, gs, ref["scores"], bound, nb, c.top_k, keep_sink, keep_local)
    return ref, same


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_select_index(name, kw):
    c = make_index_case(seed=41, **kw)
    gi, gs, qs, ks = run_index(c)
    ref, same = full_check(c, gi, gs, qs, ks)
    # every planted block scores far above the rest of its row: the GPU keeps it
    for (b, g), blocks in c.planted.items():
        if blocks and c.top_k >= len(blocks):
            assert set(blocks) <= set(gi[b, g].tolist()), (b, g)


def test_select_index_scores_optional():
    c = make_index_case(seed=42, B=2, Hkv=4, lens=[9000, 3000], top_k=16, dtype="bf16", permute=True)
    gi, _, _, _ = run_index(c, scores=False)
    gi2, _, _, _ = run_index(c)
    np.testing.assert_array_equal(gi, gi2)


def test_select_index_bad_pages_and_wide_window():
    """Page ids outside [0, num_pages) score -inf and are never read; max_seq_len past every
    length leaves -inf columns; a sequence of length 0 selects nothing."""
    c = make_index_case(seed=43, B=3, Hkv=4, lens=[6000, 2000, 0], top_k=12, dtype="f32", permute=True)
    table = c.block_table.copy()
    table[0, 3] = -1
    table[0, 50] = c.num_pages + 5
    table[1, 0] = -7
    max_len = c.max_blocks * 64
    gi, gs, qs, ks = run_index(c, max_len=max_len, table=table)
    assert np.isneginf(gs[0, :, 3]).all() and np.isneginf(gs[0, :, 50]).all() and np.isneginf(gs[1, :, 0]).all()
    full_check(c, gi, gs, qs, ks, table=table)
    assert (gi[2] == -1).all()


def test_select_index_all_tied():
    """All index keys zero: every valid score is 0 (the padded tail holds large values and must
    not be read), so the k lowest block ids win in every row."""
    c = make_index_case(seed=44, B=2, Hkv=2, lens=[64 * 37 + 5, 64 * 9 + 63], top_k=10, dtype="bf16",
                        plant=None)
    keys = np.zeros_like(c.index_keys)
    for b in range(c.B):
        n = int(c.seq_lens[b])
        keys[c.block_table[b, (n - 1) // 64], n % 64:, :] = 1000.0
    c.index_keys = keys
    gi, gs, qs, ks = run_index(c)
    for b in range(c.B):
        nb = (int(c.seq_lens[b]) + 63) // 64
        assert (gs[b, :, :nb] == 0).all()
        for g in range(c.Hkv):
            np.testing.assert_array_equal(gi[b, g], np.arange(10))
    full_check(c, gi, gs, qs, ks)


def test_select_index_full_size_1m():
    """1M cached tokens, 8 groups, k = 64, permuted pages: every score and every list is checked
    against the oracle."""
    c = make_index_case_torch(seed=45, B=1, Hkv=8, lens=[1048576], top_k=64, dtype="bf16", permute=True,
                              plant=("count", 16))
    gi, gs, qs, ks = run_index(c)
    ref, same = full_check(c, gi, gs, qs, ks)
    for (b, g), blocks in c.planted.items():
        assert set(blocks) <= set(gi[b, g].tolist()), (b, g)
