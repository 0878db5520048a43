"""Seeded random sweep of small configurations against the oracle, through the C ABI: storage type,
KV heads (powers of two and not), group size 1..8, batch, ragged lengths (0 included), k from 1 to
past the number of blocks, forced sink / local blocks, the summary pool type and page
permutation, for decode steps and prefill chunks. Each case is small; together they reach
combinations the hand-written cases do not."""
import numpy as np
import pytest

from synth import make_decode_case, make_prefill_case
from gpu_util import full_decode_check, require_gpu, run_decode, to_device

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
    kw, sink, local, sdt = decode_params(i)
    c = make_decode_case(seed=9100 + i, **kw)
    if sdt == "bf16":
        import test_gpu_bf16_summaries as tb
        d = tb.to_device_bf16(c)
        d.cfg.keep_sink, d.cfg.keep_local = sink, local
        tb.check_decode_bf16(d, run_decode(d))
    else:
        d = to_device(c)
        d.cfg.keep_sink, d.cfg.keep_local = sink, local
        full_decode_check(d, run_decode(d))


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
