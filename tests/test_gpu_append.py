"""GPU parity of the decode step's token append against the CPU oracle, through the C ABI.

msa_decode_step with k_new / v_new writes the new token's K/V row at position seq_len-1 of its
block, recomputes that block's summary from the block's keys and scores the block from the stored
summary, in the same launch as the scoring of every other block. Checked here:
  * the pools after the step equal the pools before with exactly those rows replaced (bit for
    bit; a sequence of length 0, or whose last block has an invalid page id, is left alone);
  * every stored summary against the oracle's summaries of the cache after the append (fp32
    pool: the fp32 mean's error bound; bf16 pool: one bf16 step on top of it);
  * scores, index sets, outputs and lse against the oracle run on the cache after the append,
    under the decode tolerances.
Cases cover fp32 and bf16 K/V, both summary pool types, power-of-two and other KV head counts,
the new token as the first, a middle and the last row of its block, one-token sequences, an
empty sequence, and each selection path of the top-k kernel (bound, every block kept, large k)."""
import numpy as np
import pytest
import torch

import long_context_sparse_select_amd as msa
import oracle
from synth import make_decode_case, storage
from gpu_util import dev_tensor, full_decode_check, host_store, require_gpu, run_decode, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def new_token(c, seed):
    """a seeded new token: K and V rows [B][Hkv][128] in the cache's storage type, on the device"""
    r = np.random.default_rng(seed)
    kn = r.standard_normal((c.B, c.Hkv, c.D), dtype=np.float32) * 3
    vn = r.standard_normal((c.B, c.Hkv, c.D), dtype=np.float32)
    return dev_tensor(storage(kn, c.dtype)), dev_tensor(storage(vn, c.dtype))


def check_appended_pools(d, kn, vn, k_before, v_before, table=None):
    """pools after the step == pools before with row seq_len-1 of each sequence replaced by the new
    token (where that block's page id is valid), bit for bit"""
    c = d.case
    table = c.block_table if table is None else table
    k2, v2 = k_before.copy(), v_before.copy()
    kh, vh = host_store(kn), host_store(vn)
    for b in range(c.B):
        N = min(int(c.seq_lens[b]), c.max_seq_len)
        if N == 0:
            continue
        page = int(table[b, (N - 1) // 64])
        if 0 <= page < c.num_pages:
            k2[page, :, (N - 1) % 64] = kh[b]
            v2[page, :, (N - 1) % 64] = vh[b]
    np.testing.assert_array_equal(host_store(d.k), k2)
    np.testing.assert_array_equal(host_store(d.v), v2)


def check_f32_summaries(d):
    """every stored fp32 summary within the fp32 mean's error bound (plus its own rounding) of the
    oracle's exact mean over the cache as it now is"""
    import test_gpu_bf16_summaries as tb
    c = d.case
    k_now = host_store(d.k)
    S_ref = oracle.summaries(k_pool=k_now, block_table=c.block_table, seq_lens=c.seq_lens, Hkv=c.Hkv, D=c.D, P=c.P)
    err = tb.fp32_mean_error(k_now, c.block_table, c.seq_lens, c.Hkv, c.D, S_ref.shape[1])
    S = host_store(d.S).astype(np.float64)
    for b in range(c.B):
        nb = (int(c.seq_lens[b]) + 63) // 64
        diff = np.abs(S[c.block_table[b, :nb]] - S_ref[b, :nb])
        assert np.all(diff <= err[b, :nb] + 2.0 ** -24 * np.abs(S_ref[b, :nb])), "summary off (b=%d)" % b


def device_case(c, pool):
    import test_gpu_bf16_summaries as tb
    return tb.to_device_bf16(c) if pool == "bf16" else to_device(c)


def step_and_check(d, pool, seed, sink=0, local=0, append=True):
    """one decode step with a new token (or without, append=False), then every check of the
    module docstring"""
    import test_gpu_bf16_summaries as tb
    d.cfg.keep_sink, d.cfg.keep_local = sink, local
    if append:
        k_before, v_before = host_store(d.k), host_store(d.v)
        kn, vn = new_token(d.case, seed)
        res = run_decode(d, k_new=kn, v_new=vn)
        check_appended_pools(d, kn, vn, k_before, v_before)
    else:
        res = run_decode(d)
    if pool == "bf16":
        tb.check_decode_bf16(d, res)          # includes the stored-summary check
    else:
        check_f32_summaries(d)
        full_decode_check(d, res)
    # the same step again with its scores in a workspace full of NaN bytes (so written only up to
    # each sequence's length, and never read further): the append is idempotent, so the outputs,
    # lse and lists must be bit-identical
    c = d.case
    ws = torch.full((msa.msa_workspace_size(d.cfg, msa.MSA_OP_DECODE, c.B, c.max_seq_len),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d.q)
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    idx = torch.empty((c.B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
    msa.msa_decode_step(d.cfg, d.q, d.cache, c.B, c.max_seq_len, out, k_new=kn if append else None,
                        v_new=vn if append else None, idx_out=idx, lse_out=lse, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, res["o"]) and torch.equal(lse, res["lse"]) and torch.equal(idx, res["idx"])
    return res


CASES = [
    # (name, case kwargs, summary pool)
    ("bf16_g4_rows_0_8_63", dict(B=4, Hq=32, Hkv=8, lens=[777, 64, 4097, 1], top_k=8, dtype="bf16", permute=True),
     "f32"),
    ("f32_g2_empty_sequence", dict(B=3, Hq=4, Hkv=2, lens=[2049, 63, 0], top_k=5, dtype="f32", permute=True), "f32"),
    ("f32_three_kv_heads_bf16_pool", dict(B=2, Hq=6, Hkv=3, lens=[1000, 129], top_k=4, dtype="f32"), "bf16"),
    ("bf16_g1_five_kv_heads_bf16_pool", dict(B=2, Hq=5, Hkv=5, lens=[3333, 128], top_k=7, dtype="bf16"), "bf16"),
    ("bf16_g8_every_block_kept", dict(B=1, Hq=8, Hkv=1, lens=[640], top_k=16, dtype="bf16"), "f32"),
    ("bf16_g4_large_k", dict(B=1, Hq=8, Hkv=2, lens=[262139], top_k=1024, dtype="bf16", permute=True), "f32"),
    ("bf16_g2_batch6", dict(B=6, Hq=16, Hkv=8, lens=[70000, 4096, 65, 1, 33333, 9000], top_k=64, dtype="bf16",
                            permute=True), "bf16"),
]


@pytest.mark.parametrize("name,kw,pool", CASES, ids=[c[0] for c in CASES])
def test_decode_step_with_append(name, kw, pool):
    c = make_decode_case(seed=71, **kw)
    step_and_check(device_case(c, pool), pool, seed=72)


def test_appended_block_is_forced_local():
    c = make_decode_case(seed=73, B=3, Hq=32, Hkv=8, lens=[777, 64, 40000], top_k=8, dtype="bf16", permute=True)
    res = step_and_check(to_device(c), "f32", seed=74, sink=1, local=1)
    idx = res["idx"].cpu().numpy()
    for b in range(c.B):
        jl = (int(c.seq_lens[b]) - 1) // 64
        assert (idx[b] == jl).any(axis=1).all()


def test_consecutive_steps_fill_a_block():
    """Tokens appended one step after another (the length grows by one each time) across a block
    boundary: after every step the cache and the outputs match the oracle."""
    # the cache is laid out for lengths 193 and 4, then the steps run at 190..193 and 1..4: each
    # step's append rewrites the last block's summary, and the fourth opens block 3 of sequence 0
    c = make_decode_case(seed=75, B=2, Hq=16, Hkv=4, lens=[193, 4], top_k=4, dtype="bf16", permute=True)
    d = to_device(c)
    c.seq_lens[:] = [190, 1]
    for s in range(4):
        d.lens.copy_(torch.from_numpy(c.seq_lens))
        step_and_check(d, "f32", seed=76 + s)
        c.seq_lens += 1


def test_append_with_an_invalid_last_page_id():
    """A sequence whose last block has an out-of-range page id gets nothing written, and that block
    scores -inf and is never selected; the other sequence appends normally."""
    c = make_decode_case(seed=77, B=2, Hq=8, Hkv=2, lens=[1000, 1000], top_k=4, dtype="bf16")
    d = to_device(c)
    jl = (1000 - 1) // 64
    bad = c.block_table.copy()
    bad[0, jl] = c.num_pages + 5
    d.table.copy_(torch.from_numpy(bad))
    k_before, v_before, S_before = host_store(d.k), host_store(d.v), host_store(d.S)
    kn, vn = new_token(c, 78)
    res = run_decode(d, k_new=kn, v_new=vn)
    check_appended_pools(d, kn, vn, k_before, v_before, table=bad)
    s = res["scores"].cpu().numpy()
    assert np.isneginf(s[0, :, jl]).all()
    assert not (res["idx"].cpu().numpy()[0] == jl).any()
    S_now = host_store(d.S)
    np.testing.assert_array_equal(S_now[bad[0, :jl]], S_before[bad[0, :jl]])     # sequence 0: untouched
    assert not np.array_equal(S_now[bad[1, jl]], S_before[bad[1, jl]])          # sequence 1: recomputed


def test_graph_replays_of_a_step_with_append():
    """The step with an append captured in a HIP graph: every replay (same token, same length)
    rewrites the same row and gives the eager call's outputs exactly."""
    c = make_decode_case(seed=79, B=2, Hq=32, Hkv=8, lens=[20000, 3000], top_k=32, dtype="bf16", permute=True)
    d = to_device(c)
    kn, vn = new_token(c, 80)
    out = torch.empty_like(d.q)
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    idx = torch.empty((c.B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(msa.msa_workspace_size(d.cfg, msa.MSA_OP_DECODE, c.B, c.max_seq_len), dtype=torch.uint8,
                     device="cuda")

    def step():
        msa.msa_decode_step(d.cfg, d.q, d.cache, c.B, c.max_seq_len, out, k_new=kn, v_new=vn, idx_out=idx,
                            lse_out=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    want = (out.clone(), lse.clone(), idx.clone(), d.S.clone())
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
        assert torch.equal(d.S, want[3]), r
        step()
        torch.cuda.synchronize()
