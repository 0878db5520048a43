"""Seeded random sweep of small configurations against the oracle, through the C ABI: storage type,
KV heads (powers of two and not), group size 1..8, batch, ragged lengths (0 included), k from 1 to
past the number of blocks, forced sink / local blocks, the summary pool type, page permutation
and (decode) a new token appended by the step, for decode steps and prefill chunks. Each case is small; together they reach
combinations the hand-written cases do not."""
import numpy as np
import pytest

from synth import make_decode_case, make_prefill_case
from gpu_util import require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def decode_params(i):
    r = np.random.default_rng(9000 + i)
    Hkv = int(r.choice([1, 2, 3, 4, 5, 8, 16]))
    G = int(r.integers(1, 9))
    B = int(r.integers(1, 6))
    lens = [int(x) for x in r.integers(0, 20000, size=B)]
    if r.random() < 0.3:
        lens[int(r.integers(B))] = int(r.integers(1, 130))      # a very short sequence
    sink, local = int(r.integers(0, 3)), int(r.integers(0, 3))
    k = int(max(sink + local, 1, r.integers(1, 400)))
    return dict(B=B, Hq=Hkv * G, Hkv=Hkv, lens=lens, top_k=k, dtype=str(r.choice(["f32", "bf16"])),
                permute=bool(r.random() < 0.5), plant=("count", int(r.integers(0, 4)))), sink, local, \
        str(r.choice(["f32", "bf16"]))


@pytest.mark.parametrize("i", range(48))
def test_random_decode(i):
    import test_gpu_append as ta
    kw, sink, local, sdt = decode_params(i)
    append = bool(np.random.default_rng(9050 + i).random() < 0.5)   # its own stream: the cases stay as they were
    c = make_decode_case(seed=9100 + i, **kw)
    ta.step_and_check(ta.device_case(c, sdt), sdt, seed=9060 + i, sink=sink, local=local, append=append)


def prefill_params(i):
    r = np.random.default_rng(9500 + i)
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.integers(1, 9))
    past = 64 * int(r.integers(0, 64))
    T = int(r.integers(1, 300))
    sink, local = int(r.integers(0, 2)), int(r.integers(0, 2))
    k = int(max(sink + local, 1, r.integers(1, 40)))
    return dict(Hq=Hkv * G, Hkv=Hkv, past_len=past, T=T, top_k=k), sink, local, str(r.choice(["f32", "bf16"]))


@pytest.mark.parametrize("i", range(24))
def test_random_prefill(i):
    import test_gpu_prefill as tp
    kw, sink, local, sdt = prefill_params(i)
    p = make_prefill_case(seed=9600 + i, dtype="bf16", permute=bool(i % 2), **kw)
    d = tp.to_dev(p, keep_sink=sink, keep_local=local, summary_dtype=sdt)
    k_before, v_before = tp.host_store(d["k"]), tp.host_store(d["v"])
    res = tp.run_prefill(p, d)
    tp.check_prefill(p, d, res, k_before, v_before)


@pytest.mark.parametrize("i", range(16))
def test_random_index_select(i):
    import test_gpu_index as ti
    import torch
    import long_context_sparse_select_amd as msa
    from synth import make_index_case
    r = np.random.default_rng(9800 + i)
    Hkv = int(r.choice([1, 2, 3, 4, 8, 16]))
    B = int(r.integers(1, 5))
    lens = [int(x) for x in r.integers(0, 30000, size=B)]
    sink, local = int(r.integers(0, 3)), int(r.integers(0, 3))
    k = int(max(sink + local, 1, r.integers(1, 600)))
    c = make_index_case(seed=9900 + i, B=B, Hkv=Hkv, lens=lens, top_k=k, dtype=str(r.choice(["f32", "bf16"])),
                        permute=bool(r.random() < 0.5), plant=("count", int(r.integers(0, 4))),
                        Di=int(r.choice([64, 128])))
    table = c.block_table.copy()
    if r.random() < 0.5 and c.num_pages > 4:       # a few bad page ids inside the sequences
        for _ in range(3):
            b = int(r.integers(B))
            nb = (lens[b] + 63) // 64
            if nb:
                table[b, int(r.integers(nb))] = int(r.choice([-1, c.num_pages + 3]))
    cfg, qi, ik, tab, ln = ti.device_case(c)
    cfg.keep_sink, cfg.keep_local = sink, local
    tab = torch.from_numpy(np.ascontiguousarray(table)).cuda()
    mb = (c.max_seq_len + 63) // 64
    idx = torch.empty((c.B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
    sc = torch.full((c.B, c.Hkv, max(mb, 1)), float("nan"), dtype=torch.float32, device="cuda")
    msa.msa_select_index(cfg, qi, ik, tab, ln, c.B, c.max_seq_len, idx, scores_out=sc)
    torch.cuda.synchronize()
    ti.full_check(c, idx.cpu().numpy(), sc.cpu().numpy()[:, :, :mb], ti.host_store(qi), ti.host_store(ik),
                  table=table, keep_sink=sink, keep_local=local)


@pytest.mark.parametrize("i", range(12))
def test_random_attend_on_caller_lists(i):
    """msa_attend over caller-supplied lists that mix valid ids with -1 and out-of-range entries
    (skipped), against the oracle attending the same lists."""
    import torch
    import long_context_sparse_select_amd as msa
    import oracle
    from gpu_util import assert_close, host_f64, oracle_inputs
    kw, _, _, _ = decode_params(100 + i)
    c = make_decode_case(seed=9700 + i, **kw)
    d = to_device(c)
    r = np.random.default_rng(9750 + i)
    idx = np.full((c.B, c.Hkv, c.top_k), -1, np.int32)
    for b in range(c.B):
        nb = (int(c.seq_lens[b]) + 63) // 64
        for g in range(c.Hkv):
            m = int(r.integers(0, min(c.top_k, nb) + 1)) if nb else 0
            sel = r.choice(nb, size=m, replace=False) if m else np.zeros(0, np.int64)
            row = list(sel) + [int(x) for x in r.choice([-1, -5, nb, nb + 7], size=c.top_k - m)]
            r.shuffle(row)
            idx[b, g] = row
    out = torch.empty_like(d.q)
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    msa.msa_attend(d.cfg, d.q, d.cache, c.B, c.max_seq_len, torch.from_numpy(idx).cuda(), out, lse_out=lse)
    torch.cuda.synchronize()
    ref = oracle.decode(idx_in=idx, **oracle_inputs(d))
    assert_close(host_f64(out), ref["o"], c.dtype, "o")
    assert_close(lse.cpu().numpy(), ref["lse"], c.dtype, "lse", lse=True)
