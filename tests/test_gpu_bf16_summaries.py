"""GPU parity of the bf16 summary pool (each summary is its block's mean rounded to bf16, ties to
even; every score uses the stored bf16 summary) against the CPU oracle, through the C ABI.

Tolerance: the oracle rounds the exact mean once; the GPU rounds its fp32 mean, which can land on
the neighbouring bf16 value when the exact mean sits next to a rounding boundary, or further when
the fp32 sum's own error exceeds the bf16 step of a near-zero mean (fp32 keys). Each stored
summary must therefore lie within one bf16 step plus the fp32 mean's error bound of the rounded
mean, and a block's score may move by the observed difference
E_j = sum_d |q_idx,d| * |S_gpu,j,d - S_ref,j,d| on top of the fp32 arithmetic term of the fp32 pool.
The index-set band widens by max_j E_j for the same reason.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_select_amd as msa
import oracle
from synth import make_decode_case, make_decode_case_torch, make_prefill_case, round_to_bf16, storage
from gpu_util import (Dev, SCORE_RTOL, assert_close, bf16_step, check_index_sets, dev_tensor, host_f64,
                      host_store, oracle_inputs, require_gpu, run_decode)
from helpers import as_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def to_device_bf16(case) -> Dev:
    if isinstance(case.q, torch.Tensor):
        q, k, v = case.q, case.k_pool, case.v_pool
    else:
        q, k, v = (dev_tensor(storage(x, case.dtype)) for x in (case.q, case.k_pool, case.v_pool))
    table = torch.from_numpy(np.ascontiguousarray(case.block_table)).cuda()
    lens = torch.from_numpy(np.ascontiguousarray(case.seq_lens)).cuda()
    S = torch.full((case.num_pages, case.Hkv, case.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    cfg = msa.make_config(case.Hq, case.Hkv, case.top_k, dtype=case.dtype, softmax_scale=case.scale,
                          summary_dtype="bf16")
    cache = msa.KVCache(k, v, S, table, lens)
    msa.msa_build_summaries(cfg, cache, case.B, case.max_seq_len)
    return Dev(case, q, k, v, table, lens, S, cfg, cache)


def fp32_mean_error(k_store, table, lens, Hkv, D, mb):
    """Bound on |fp32 mean - exact mean| of each block summary: (n + 2) * 2^-24 * sum_t |k_t| / n
    over the block's n valid keys (fp32 summation and the division). [B][mb][Hkv][D]."""
    ak = np.abs(as_f64(k_store)).astype(np.float32)
    out = np.zeros((len(lens), mb, Hkv, D))
    for b, N in enumerate(lens):
        N = int(N)
        nb = (N + 63) // 64
        full = N // 64
        if full:
            out[b, :full] = ak[table[b, :full]].sum(axis=2, dtype=np.float64) * (66.0 / 64.0)
        if nb > full:
            n = N - 64 * full
            out[b, full] = ak[table[b, full], :, :n].sum(axis=1, dtype=np.float64) * ((n + 2.0) / n)
    return out * 2.0 ** -24


def summary_check(d, inputs):
    """Stored bf16 summaries against the oracle's rounded means: returns (S_ref, |S_gpu - S_ref|)
    as [B][max_blocks][Hkv][D] (zero past each sequence's blocks). Both sides round monotonically,
    so they differ by at most the fp32 mean's own error plus one bf16 step at the larger value."""
    c = d.case
    S_ref = oracle.summaries(k_pool=inputs["k_pool"], block_table=c.block_table, seq_lens=c.seq_lens, Hkv=c.Hkv,
                             D=c.D, P=c.P, summary_dtype="bf16")
    err = fp32_mean_error(inputs["k_pool"], c.block_table, c.seq_lens, c.Hkv, c.D, S_ref.shape[1])
    S_gpu = host_f64(d.S)
    diff = np.zeros_like(S_ref)
    for b in range(c.B):
        nb = (int(c.seq_lens[b]) + 63) // 64
        g = S_gpu[c.block_table[b, :nb]]
        diff[b, :nb] = np.abs(g - S_ref[b, :nb])
        allowed = bf16_step(np.maximum(np.abs(S_ref[b, :nb]), np.abs(g))) + err[b, :nb]
        assert np.all(diff[b, :nb] <= allowed), "a summary is beyond one bf16 step + fp32 error (b=%d)" % b
    return S_ref, diff


def check_decode_bf16(d, res):
    c = d.case
    inputs = oracle_inputs(d)
    ref = oracle.decode(summary_dtype="bf16", **inputs)
    S_ref, diff = summary_check(d, inputs)
    G = c.Hq // c.Hkv
    mb = res["scores"].shape[2]
    qidx = np.abs(host_f64(d.q).reshape(c.B, c.Hkv, G, c.D).mean(axis=2))          # [B][Hkv][D]
    A = np.einsum("bgd,bjgd->bgj", qidx, np.abs(S_ref[:, :mb]))
    E = np.einsum("bgd,bjgd->bgj", qidx, diff[:, :mb])
    nb = (c.seq_lens.astype(np.int64) + 63) // 64
    gs = res["scores"].cpu().numpy()
    for b in range(c.B):
        n = int(nb[b])
        r_s, g_s = ref["scores"][b, :, :n], gs[b, :, :n].astype(np.float64)
        tol = SCORE_RTOL * np.maximum(np.abs(r_s), A[b, :, :n]) + E[b, :, :n]
        assert np.all(np.abs(g_s - r_s) <= tol), "score mismatch b=%d" % b
        assert np.all(np.isneginf(gs[b, :, n:]))
    gi = res["idx"].cpu().numpy()
    slack = np.array([[E[b, g, :int(nb[b])].max() if nb[b] else 0.0 for g in range(c.Hkv)] for b in range(c.B)])
    same = check_index_sets(gi, gs, ref["scores"], A, nb, c.top_k, inputs["keep_sink"], inputs["keep_local"],
                            slack=slack)
    if not same.all():
        ref = oracle.decode(idx_in=gi, summary_dtype="bf16", **inputs)
    assert_close(host_f64(res["o"]), ref["o"], c.dtype, "o")
    assert_close(res["lse"].cpu().numpy(), ref["lse"], c.dtype, "lse", lse=True)
    return int((~same).sum()), int((diff > 0).sum())


CASES = [
    ("bf16_g4_ragged", dict(B=3, Hq=32, Hkv=8, lens=[8192, 5000, 131], top_k=32, dtype="bf16",
                            plant=("frac", 0.01), permute=True)),
    ("f32_kv_g2_tail", dict(B=2, Hq=4, Hkv=2, lens=[2049, 63], top_k=5, dtype="f32", permute=True)),
    ("bf16_g8_bigk", dict(B=1, Hq=16, Hkv=2, lens=[20000], top_k=300, dtype="bf16")),
    ("bf16_g1_odd_heads", dict(B=2, Hq=6, Hkv=6, lens=[3333, 700], top_k=7, dtype="bf16")),
    ("bf16_g2_wide", dict(B=6, Hq=16, Hkv=8, lens=[70000, 4096, 65, 1, 33333, 9000], top_k=64, dtype="bf16",
                          permute=True)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_decode_step_bf16_summaries(name, kw):
    c = make_decode_case(seed=61, **kw)
    d = to_device_bf16(c)
    check_decode_bf16(d, run_decode(d))


def test_select_and_score_entry_points_bf16_summaries():
    c = make_decode_case(seed=62, B=2, Hq=32, Hkv=8, lens=[9000, 3000], top_k=16, dtype="bf16", permute=True)
    d = to_device_bf16(c)
    mb = (c.max_seq_len + 63) // 64
    s1 = torch.full((c.B, c.Hkv, mb), float("nan"), dtype=torch.float32, device="cuda")   # every entry written
    s2 = torch.full_like(s1, float("nan"))
    idx = torch.empty((c.B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
    msa.msa_score(d.cfg, d.q, d.cache, c.B, c.max_seq_len, s1)
    msa.msa_select(d.cfg, d.q, d.cache, c.B, c.max_seq_len, idx, scores_out=s2)
    torch.cuda.synchronize()
    assert not torch.isnan(s1).any() and not torch.isnan(s2).any()
    np.testing.assert_array_equal(s1.cpu().numpy(), s2.cpu().numpy())
    res = run_decode(d)
    np.testing.assert_array_equal(res["idx"].cpu().numpy(), idx.cpu().numpy())


def test_decode_step_appends_into_a_bf16_pool():
    """The step's append rewrites the last block's bf16 summary and scores it from the stored value."""
    c = make_decode_case(seed=63, B=3, Hq=32, Hkv=8, lens=[777, 64, 4097], top_k=8, dtype="bf16", permute=True)
    d = to_device_bf16(c)
    r = np.random.default_rng(9)
    kn = round_to_bf16(r.standard_normal((c.B, c.Hkv, c.D), dtype=np.float32) * 3)
    vn = round_to_bf16(r.standard_normal((c.B, c.Hkv, c.D), dtype=np.float32))
    res = run_decode(d, k_new=dev_tensor(storage(kn, "bf16")), v_new=dev_tensor(storage(vn, "bf16")))
    check_decode_bf16(d, res)   # the oracle reads the cache after the append


def test_full_size_decode_1m_bf16_summaries():
    """The 1M-token workload with a bf16 pool: every score, list and output against the oracle."""
    c = make_decode_case_torch(seed=64, B=1, Hq=32, Hkv=8, lens=[1048576], top_k=64, dtype="bf16", permute=True,
                               plant=("count", 16), device="cuda")
    d = to_device_bf16(c)
    check_decode_bf16(d, run_decode(d))


PREFILL = [
    ("past640_T200", dict(Hq=32, Hkv=8, past_len=640, T=200, top_k=3)),
    ("past4096_T256_g8", dict(Hq=8, Hkv=1, past_len=4096, T=256, top_k=16)),
]


@pytest.mark.parametrize("name,kw", PREFILL, ids=[c[0] for c in PREFILL])
def test_prefill_chunk_bf16_summaries(name, kw):
    import test_gpu_prefill as tp
    p = make_prefill_case(seed=65, dtype="bf16", permute=True, **kw)
    d = tp.to_dev(p, summary_dtype="bf16")
    k_before, v_before = host_store(d["k"]), host_store(d["v"])
    res = tp.run_prefill(p, d)
    tp.check_prefill(p, d, res, k_before, v_before)
