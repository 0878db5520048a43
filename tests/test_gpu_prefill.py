"""GPU parity of the prefill chunk (append + summaries, tile scoring, top-k + diagonal block,
MFMA causal attention) against the CPU oracle, through the C ABI. Small cases span several
tiles with ragged tails and every group size path; the full 4096-on-262144 chunk is checked on
sampled tiles."""
import numpy as np
import pytest
import torch

import long_context_sparse_select_amd as msa
import oracle
from synth import bf16_bits_to_f32, make_prefill_case, make_prefill_case_torch, storage, workload
from gpu_util import (SCORE_RTOL, assert_close, bf16_step, check_band, dev_tensor, host_f64, host_store, require_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def to_dev(p, keep_sink=0, keep_local=0, summary_dtype="f32"):
    if isinstance(p.q, torch.Tensor):
        q, kn, vn, k, v = p.q, p.k_new, p.v_new, p.k_pool, p.v_pool
    else:
        q, kn, vn, k, v = (dev_tensor(storage(x, p.dtype)) for x in (p.q, p.k_new, p.v_new, p.k_pool, p.v_pool))
    table = torch.from_numpy(p.block_table).cuda()
    sdt = torch.bfloat16 if summary_dtype == "bf16" else torch.float32
    S = torch.full((p.num_pages, p.Hkv, p.D), float("nan"), dtype=sdt, device="cuda")
    lens = torch.tensor([p.past_len], dtype=torch.int32, device="cuda")
    cfg = msa.make_config(p.Hq, p.Hkv, p.top_k, dtype=p.dtype, softmax_scale=p.scale, keep_sink=keep_sink,
                          keep_local=keep_local, summary_dtype=summary_dtype)
    cache = msa.KVCache(k, v, S, table, lens)
    if p.past_len:
        msa.msa_build_summaries(cfg, cache, 1, p.past_len)
    return dict(q=q, kn=kn, vn=vn, k=k, v=v, table=table, S=S, cfg=cfg, cache=cache)


def run_prefill(p, d):
    ntiles = (p.T + 63) // 64
    mb = p.past_len // 64 + ntiles
    out = torch.empty_like(d["q"])
    lse = torch.empty((p.T, p.Hq), dtype=torch.float32, device="cuda")
    idx = torch.empty((ntiles, p.Hkv, p.top_k + 1), dtype=torch.int32, device="cuda")
    scores = torch.empty((ntiles, p.Hkv, mb), dtype=torch.float32, device="cuda")
    msa.msa_prefill_chunk(d["cfg"], d["q"], d["kn"], d["vn"], d["cache"], p.past_len, p.T, out, idx_out=idx,
                          scores_out=scores, lse_out=lse)
    torch.cuda.synchronize()
    return dict(o=out, lse=lse, idx=idx.cpu().numpy(), scores=scores.cpu().numpy())


def block_means(p, k_pool_store, kn_store, absolute=False):
    """[blocks][Hkv][D] fp64 means of the keys of the sequence after the chunk is appended (of their
    magnitudes with absolute=True)."""
    f = np.abs if absolute else (lambda x: x)
    past_blocks, ntiles = p.past_len // 64, (p.T + 63) // 64
    out = np.empty((past_blocks + ntiles, p.Hkv, p.D))
    for g in range(p.Hkv):
        if past_blocks:
            blk = bf16_bits_to_f32(k_pool_store[p.block_table[0, :past_blocks], g]).astype(np.float64)
            out[:past_blocks, g] = f(blk).mean(axis=1)
    kn = bf16_bits_to_f32(kn_store).astype(np.float64)
    for jn in range(ntiles):
        out[past_blocks + jn] = f(kn[jn * 64:min(p.T, jn * 64 + 64)]).mean(axis=0)
    return out


def check_prefill(p, d, res, k_pool_before, v_pool_before, tiles=None):
    """scores (fp32 tolerance), selection (exact on the GPU's scores + band), outputs."""
    ntiles = (p.T + 63) // 64
    lo, hi = tiles if tiles is not None else (0, ntiles)
    sd = "bf16" if int(d["cfg"].summary_dtype) == msa.MSA_BF16 else "f32"
    kw = dict(q=host_store(d["q"]), k_new=host_store(d["kn"]), v_new=host_store(d["vn"]),
              k_pool=k_pool_before, v_pool=v_pool_before, block_table=p.block_table,
              past_len=p.past_len, Hq=p.Hq, Hkv=p.Hkv, top_k=p.top_k, scale=p.scale, P=p.P,
              keep_sink=int(d["cfg"].keep_sink), keep_local=int(d["cfg"].keep_local), summary_dtype=sd)
    ref = oracle.prefill(tiles=(lo, hi), **kw)
    G = p.Hq // p.Hkv
    q64 = host_f64(d["q"])
    S64 = block_means(p, k_pool_before, host_store(d["kn"]))   # fp64 means, for the tolerance scale
    # bf16 pool: the GPU's stored summaries against the rounded means (both round monotonically,
    # so they differ by at most one bf16 step plus the fp32 mean's error, (n + 2) 2^-24 mean|k|);
    # their difference bounds the extra score error of each block
    diff = np.zeros_like(S64)
    if sd == "bf16":
        S_ref = torch.from_numpy(S64).to(torch.bfloat16).to(torch.float64).numpy()
        S_gpu = host_f64(d["S"])[p.block_table[0, :S64.shape[0]]]
        diff = np.abs(S_gpu - S_ref)
        err = block_means(p, k_pool_before, host_store(d["kn"]), absolute=True) * 66.0 * 2.0 ** -24
        allowed = bf16_step(np.maximum(np.abs(S_ref), np.abs(S_gpu))) + err
        assert np.all(diff <= allowed), "a bf16 summary is beyond one bf16 step + fp32 error of the rounded mean"
    same_all = True
    for tau in range(lo, hi):
        rows = slice(tau * 64, min(p.T, tau * 64 + 64))
        n = p.past_len // 64 + tau
        keff = min(p.top_k, n)
        for g in range(p.Hkv):
            qt = q64[rows, g * G:(g + 1) * G].reshape(-1, p.D).mean(axis=0)
            bound = np.abs(S64[:n, g]) @ np.abs(qt)
            extra = diff[:n, g] @ np.abs(qt)
            r_s = ref["scores"][tau, g, :n]
            g_s = res["scores"][tau, g, :n].astype(np.float64)
            tol = SCORE_RTOL * np.maximum(np.abs(r_s), bound) + extra
            assert np.all(np.abs(g_s - r_s) <= tol), "prefill score mismatch tau=%d g=%d" % (tau, g)
            assert np.all(np.isneginf(res["scores"][tau, g, n:]))
            sel = res["idx"][tau, g]
            want = oracle.topk(g_s, p.top_k, keep_sink=kw["keep_sink"], keep_local=kw["keep_local"])
            np.testing.assert_array_equal(sel[:keff], want[:keff])
            assert sel[keff] == n and np.all(sel[keff + 1:] == -1)
            if keff:
                check_band(sel[:keff], r_s, keff, float(bound.max()), kw["keep_sink"], kw["keep_local"],
                           "(tau=%d g=%d)" % (tau, g), float(extra.max()) if n else 0.0)
            same_all &= bool(np.array_equal(sel, ref["idx"][tau, g]))
    if not same_all:
        ref = oracle.prefill(tiles=(lo, hi), idx_in=res["idx"], **kw)
    rows = slice(lo * 64, min(p.T, hi * 64))
    assert_close(host_f64(res["o"])[rows], ref["o"][rows], "bf16", "prefill o")
    assert_close(res["lse"].cpu().numpy()[rows], ref["lse"][rows], "bf16", "prefill lse", lse=True)


SMALL = [
    ("past256_T128_g4", dict(Hq=8, Hkv=2, past_len=256, T=128, top_k=2)),
    ("past640_T200_g4_ragged", dict(Hq=32, Hkv=8, past_len=640, T=200, top_k=3)),
    ("past0_T130_g4", dict(Hq=8, Hkv=2, past_len=0, T=130, top_k=4)),
    ("past1024_T64_g3", dict(Hq=6, Hkv=2, past_len=1024, T=64, top_k=5)),
    ("past4096_T256_g8", dict(Hq=8, Hkv=1, past_len=4096, T=256, top_k=16)),
    ("past128_T1_g1", dict(Hq=4, Hkv=4, past_len=128, T=1, top_k=2)),
    ("past2048_T300_g2_bigk", dict(Hq=4, Hkv=2, past_len=2048, T=300, top_k=40)),
    # short chunks on long caches: each tile's list split over several workgroups (4 and 4, the
    # second with the group's 8 heads over two workgroups as well), partials merged
    ("past65536_T512_g4_split", dict(Hq=32, Hkv=8, past_len=65536, T=512, top_k=32)),
    ("past8192_T200_g8_split", dict(Hq=64, Hkv=8, past_len=8192, T=200, top_k=24)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_prefill_chunk(name, kw):
    p = make_prefill_case(seed=41, dtype="bf16", permute=True, **kw)
    d = to_dev(p)
    k_before, v_before = host_store(d["k"]), host_store(d["v"])
    res = run_prefill(p, d)
    # the chunk landed in its pages
    k_after, v_after = host_store(d["k"]), host_store(d["v"])
    kn, vn = storage(p.k_new, "bf16"), storage(p.v_new, "bf16")
    for i in range(p.T):
        t = p.past_len + i
        pg = p.block_table[0, t // 64]
        np.testing.assert_array_equal(k_after[pg, :, t % 64], kn[i])
        np.testing.assert_array_equal(v_after[pg, :, t % 64], vn[i])
    # summaries of the new blocks
    S = d["S"].cpu().numpy()
    for jn in range((p.T + 63) // 64):
        rows = slice(jn * 64, min(p.T, jn * 64 + 64))
        want = host_f64(d["kn"])[rows].mean(axis=0)           # [Hkv][D]
        got = S[p.block_table[0, p.past_len // 64 + jn]]
        np.testing.assert_allclose(got, want, rtol=1e-5, atol=2e-6)
    check_prefill(p, d, res, k_before, v_before)


def test_prefill_deterministic():
    p = make_prefill_case(seed=42, dtype="bf16", Hq=32, Hkv=8, past_len=1280, T=256, top_k=8)
    d = to_dev(p)
    r1 = run_prefill(p, d)
    r2 = run_prefill(p, d)
    assert torch.equal(r1["o"], r2["o"]) and torch.equal(r1["lse"], r2["lse"])
    np.testing.assert_array_equal(r1["idx"], r2["idx"])


@pytest.fixture(scope="module")
def full_prefill():
    """The 4096-token chunk on a 262,144-token cache, run once on the GPU; the host copies of the
    pools from before the append feed the oracle."""
    require_gpu()
    kw = workload("prefill_bf16_4k_on_256k", seed=0)
    p = make_prefill_case_torch(**kw)
    d = to_dev(p)
    k_before, v_before = host_store(d["k"]), host_store(d["v"])
    res = run_prefill(p, d)
    return p, d, res, k_before, v_before


@pytest.mark.parametrize("tiles", [(0, 16), (16, 32), (32, 48), (48, 64)])
def test_prefill_full_size(full_prefill, tiles):
    """Every one of the 64 tiles of the full chunk, in four ranges (one oracle call each)."""
    p, d, res, k_before, v_before = full_prefill
    print("prefill 4096 on 262144: tiles %d..%d" % tiles, flush=True)
    check_prefill(p, d, res, k_before, v_before, tiles=tiles)


def test_prefill_full_size_planted(full_prefill):
    """Planted blocks are found (input-recipe sanity, not parity)."""
    p, d, res, _, _ = full_prefill
    hit = sum(int(j in res["idx"][tau, g]) for (tau, g), j in p.planted.items())
    assert hit / len(p.planted) > 0.8


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_prefill_attend_with_oracle_lists(name, kw):
    """Step 2 alone (msa_prefill_attend) over the oracle's own lists, after the chunk's append."""
    p = make_prefill_case(seed=45, dtype="bf16", permute=True, **kw)
    d = to_dev(p)
    k_before, v_before = host_store(d["k"]), host_store(d["v"])
    run_prefill(p, d)                                     # appends the chunk's K/V
    ref = oracle.prefill(q=host_store(d["q"]), k_new=host_store(d["kn"]), v_new=host_store(d["vn"]),
                         k_pool=k_before, v_pool=v_before, block_table=p.block_table, past_len=p.past_len,
                         Hq=p.Hq, Hkv=p.Hkv, top_k=p.top_k, scale=p.scale, P=p.P)
    out = torch.empty_like(d["q"])
    lse = torch.empty((p.T, p.Hq), dtype=torch.float32, device="cuda")
    idx = torch.from_numpy(ref["idx"]).cuda()
    msa.msa_prefill_attend(d["cfg"], d["q"], d["cache"], p.past_len, p.T, idx, out, lse_out=lse)
    torch.cuda.synchronize()
    assert_close(host_f64(out), ref["o"], "bf16", "prefill attend o")
    assert_close(lse.cpu().numpy(), ref["lse"], "bf16", "prefill attend lse", lse=True)


def test_prefill_graph_replays_match_eager():
    """The prefill chunk captured in a HIP graph reproduces the eager outputs on every replay (the
    append rewrites the same rows with the same values, so the chunk is idempotent)."""
    p = make_prefill_case(seed=47, dtype="bf16", permute=True, Hq=32, Hkv=8, past_len=1024, T=300, top_k=4)
    d = to_dev(p)
    ntiles = (p.T + 63) // 64
    out = torch.empty_like(d["q"])
    lse = torch.empty((p.T, p.Hq), dtype=torch.float32, device="cuda")
    idx = torch.empty((ntiles, p.Hkv, p.top_k + 1), dtype=torch.int32, device="cuda")
    ws = torch.empty(msa.msa_workspace_size(d["cfg"], msa.MSA_OP_PREFILL, 1, p.past_len + p.T, p.T),
                     dtype=torch.uint8, device="cuda")

    def chunk():
        msa.msa_prefill_chunk(d["cfg"], d["q"], d["kn"], d["vn"], d["cache"], p.past_len, p.T, out, idx_out=idx,
                              lse_out=lse, workspace=ws)

    chunk()
    torch.cuda.synchronize()
    want = (out.clone(), lse.clone(), idx.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chunk()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chunk()
    for r in range(3):
        out.zero_(); lse.zero_(); idx.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want[0]) and torch.equal(lse, want[1]) and torch.equal(idx, want[2]), r
        chunk()
        torch.cuda.synchronize()
