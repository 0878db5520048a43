"""msa_decode_step_noalloc (the decode step whose workspace is the library's own per-GPU scratch
array) against msa_decode_step with a caller workspace, through the C ABI. Both run the same
kernels on the same inputs, so their outputs must be identical; two calls in a row, the second
with a smaller input, with and without the token append, with and without the optional outputs
(without them, the lists and scores live in the scratch array too)."""
import numpy as np
import pytest
import torch

import long_context_sparse_select_amd as msa
from synth import make_decode_case, round_to_bf16, storage
from gpu_util import dev_tensor, require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _step(fn, d, c, k_new=None, v_new=None, outputs=True):
    mb = (c.max_seq_len + 63) // 64
    out = torch.full_like(d.q, float("nan"))
    lse = torch.full((c.B, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((c.B, c.Hkv, c.top_k), -7, dtype=torch.int32, device="cuda") if outputs else None
    scores = torch.full((c.B, c.Hkv, mb), float("nan"), dtype=torch.float32, device="cuda") if outputs else None
    fn(d.cfg, d.q, d.cache, c.B, c.max_seq_len, out, k_new=k_new, v_new=v_new, idx_out=idx, scores_out=scores,
       lse_out=lse)
    torch.cuda.synchronize()
    return dict(o=out, lse=lse, idx=idx, scores=scores)


def _same(a, b, what):
    for key in ("o", "lse", "idx", "scores"):
        if a[key] is None:
            continue
        x, y = a[key], b[key]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), "%s: %s differs" % (what, key)


# the first call's workspace is the larger: 3 x 70000 tokens x 8 KV heads; then a smaller one
CALLS = [
    ("bf16_b3_g4_70k", dict(B=3, Hq=32, Hkv=8, lens=[70000, 5000, 131], top_k=64, dtype="bf16", permute=True)),
    ("f32_b1_g4_3k", dict(B=1, Hq=8, Hkv=2, lens=[3000], top_k=16, dtype="f32")),
]


@pytest.mark.parametrize("outputs", [True, False])
def test_noalloc_matches_decode_step(outputs):
    for seed, (name, kw) in enumerate(CALLS):
        print("no-alloc decode step: %s, optional outputs %s" % (name, outputs), flush=True)
        c = make_decode_case(seed=70 + seed, **kw)
        d = to_device(c)
        ref = _step(msa.msa_decode_step, d, c, outputs=outputs)
        got = _step(msa.msa_decode_step_noalloc, d, c, outputs=outputs)
        _same(ref, got, name)
        assert torch.isfinite(got["o"].float()).all()


def test_noalloc_append_matches_decode_step():
    """With a new token: both entry points, each on its own copy of the cache, write the same
    K/V row and summary and return the same outputs; two calls, the second smaller."""
    for seed, (name, kw) in enumerate(CALLS):
        print("no-alloc decode step with append: %s" % name, flush=True)
        c = make_decode_case(seed=80 + seed, **kw)
        r = np.random.default_rng(seed)
        kn = dev_tensor(storage(round_to_bf16(r.standard_normal((c.B, c.Hkv, c.D), dtype=np.float32)), c.dtype))
        vn = dev_tensor(storage(round_to_bf16(r.standard_normal((c.B, c.Hkv, c.D), dtype=np.float32)), c.dtype))
        da = to_device(c)
        db = to_device(c)
        ref = _step(msa.msa_decode_step, da, c, k_new=kn, v_new=vn)
        got = _step(msa.msa_decode_step_noalloc, db, c, k_new=kn, v_new=vn)
        _same(ref, got, name)
        for t in ("k", "v", "S"):
            x, y = getattr(da, t), getattr(db, t)
            if x.dtype == torch.bfloat16:
                x, y = x.view(torch.int16), y.view(torch.int16)
            assert torch.equal(torch.nan_to_num(x.float()) if t == "S" else x,
                               torch.nan_to_num(y.float()) if t == "S" else y), "%s: cache %s differs" % (name, t)
