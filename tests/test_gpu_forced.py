"""GPU parity of forced sink / local blocks (the first keep_sink and last keep_local candidates of
every row are always kept and count toward k_eff) against the CPU oracle, through the C ABI, on
every selection path of the top-k kernel: the group-maximum bound (k <= 256), the exact large-k
select, the memory-based path for rows longer than 16,384 blocks, a step with a token append, the
prefill tiles and the index branch."""
import numpy as np
import pytest
import torch

import long_context_sparse_select_amd as msa
from synth import make_decode_case, make_decode_case_torch, make_index_case, make_prefill_case, round_to_bf16, \
    storage
from gpu_util import dev_tensor, full_decode_check, require_gpu, run_decode, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


DECODE = [
    # (name, case kwargs, keep_sink, keep_local)
    ("bf16_exactly_forced", dict(B=2, Hq=8, Hkv=2, lens=[5000, 700], top_k=2, dtype="bf16", permute=True), 1, 1),
    ("bf16_bound_path", dict(B=3, Hq=32, Hkv=8, lens=[8192, 5000, 131], top_k=32, dtype="bf16",
                             plant=("frac", 0.01), permute=True), 1, 1),
    ("f32_local2_ragged", dict(B=2, Hq=4, Hkv=2, lens=[2049, 63], top_k=5, dtype="f32", permute=True), 0, 2),
    ("bf16_large_k", dict(B=1, Hq=8, Hkv=2, lens=[262144], top_k=1024, dtype="bf16", permute=True), 2, 1),
    ("bf16_rows_sink4_local4", dict(B=6, Hq=16, Hkv=8, lens=[70000, 4096, 65, 1, 33333, 9000], top_k=64,
                                    dtype="bf16", permute=True), 4, 4),
]


def forced(d, sink, local):
    d.cfg.keep_sink = sink
    d.cfg.keep_local = local
    return d


@pytest.mark.parametrize("name,kw,sink,local", DECODE, ids=[c[0] for c in DECODE])
def test_decode_step_forced(name, kw, sink, local):
    c = make_decode_case(seed=51, **kw)
    d = forced(to_device(c), sink, local)
    res = run_decode(d)
    full_decode_check(d, res)
    idx = res["idx"].cpu().numpy()
    for b in range(c.B):
        nb = (int(c.seq_lens[b]) + 63) // 64
        for g in range(c.Hkv):
            row = set(idx[b, g].tolist())
            assert {j for j in range(nb) if j < sink or j >= nb - local} <= row


def test_decode_step_forced_with_append():
    """A step with a token append: the appended token's block is the forced local block."""
    c = make_decode_case(seed=52, B=3, Hq=32, Hkv=8, lens=[777, 64, 40000], top_k=8, dtype="bf16", permute=True)
    d = forced(to_device(c), 1, 1)
    r = np.random.default_rng(7)
    kn = round_to_bf16(r.standard_normal((c.B, c.Hkv, c.D), dtype=np.float32) * 3)
    vn = round_to_bf16(r.standard_normal((c.B, c.Hkv, c.D), dtype=np.float32))
    res = run_decode(d, k_new=dev_tensor(storage(kn, "bf16")), v_new=dev_tensor(storage(vn, "bf16")))
    full_decode_check(d, res)   # the oracle reads the cache after the append


@pytest.mark.parametrize("sink,local", [(0, 0), (1, 1)])
def test_rows_longer_than_the_register_tile(sink, local):
    """16,385 blocks in one row: the selection runs from memory (no per-thread register tile)."""
    c = make_decode_case_torch(seed=53, B=1, Hq=8, Hkv=1, lens=[16385 * 64 - 10], top_k=64, dtype="bf16",
                               permute=True, plant=("count", 16), device="cuda")
    d = forced(to_device(c), sink, local)
    res = run_decode(d)
    full_decode_check(d, res)


PREFILL = [
    ("past640_T200_sink1_local1", dict(Hq=32, Hkv=8, past_len=640, T=200, top_k=3), 1, 1),
    ("past4096_T256_sink2_local2", dict(Hq=8, Hkv=1, past_len=4096, T=256, top_k=16), 2, 2),
    ("past0_T130_sink1", dict(Hq=8, Hkv=2, past_len=0, T=130, top_k=1), 1, 0),
]


@pytest.mark.parametrize("name,kw,sink,local", PREFILL, ids=[c[0] for c in PREFILL])
def test_prefill_chunk_forced(name, kw, sink, local):
    import test_gpu_prefill as tp
    p = make_prefill_case(seed=54, dtype="bf16", permute=True, **kw)
    d = tp.to_dev(p, keep_sink=sink, keep_local=local)
    k_before, v_before = tp.host_store(d["k"]), tp.host_store(d["v"])
    res = tp.run_prefill(p, d)
    tp.check_prefill(p, d, res, k_before, v_before)


def test_index_branch_forced():
    import test_gpu_index as ti
    c = make_index_case(seed=55, B=3, Hkv=8, lens=[8192, 5000, 131], top_k=32, dtype="bf16", permute=True)
    cfg, qi, ik, tab, lens = ti.device_case(c)
    cfg.keep_sink, cfg.keep_local = 2, 1
    mb = (c.max_seq_len + 63) // 64
    idx = torch.empty((c.B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
    sc = torch.full((c.B, c.Hkv, mb), float("nan"), dtype=torch.float32, device="cuda")
    msa.msa_select_index(cfg, qi, ik, tab, lens, c.B, c.max_seq_len, idx, scores_out=sc)
    torch.cuda.synchronize()
    gi, gs = idx.cpu().numpy(), sc.cpu().numpy()
    ti.full_check(c, gi, gs, ti.host_store(qi), ti.host_store(ik), keep_sink=2, keep_local=1)
