"""GPU-side test utilities: move seeded cases to the device, run libmsa through its C ABI
(the Python binding), and compare with the oracle under the stated tolerances.

Tolerances (stated for this workload):
  * stage-1 scores (fp32): |gpu - ref| <= 1e-5 * max(|ref|, sum_d |q_idx,d * S_j,d|); the second
    term covers cancellation, where a relative bound on a near-zero score is meaningless;
  * index sets: the GPU set must equal the oracle's top-k applied to the GPU's own fp32 scores
    (same-precision decision, bit-exact), and against the fp64 oracle scores every block more
    than w = 1e-5 * max(|tau|, sum |q_idx * S|) above the k-th score tau must be in the set and
    every block more than w below it must be out;
  * outputs: |gpu - ref| <= atol + rtol * |ref| with (atol, rtol) = (2e-2, 1e-2) for bf16 and
    (1e-5, 1e-5) for fp32; lse: (1e-4, 1e-5) for bf16, (1e-5, 1e-5) for fp32. When the index sets
    differ only inside the band, the output is compared with the oracle run on the GPU's set.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import long_context_sparse_select_amd as msa
import oracle
from synth import DecodeCase, bf16_bits_to_f32, storage

OUT_TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-5, 1e-5)}
LSE_TOL = {"bf16": (1e-4, 1e-5), "f32": (1e-5, 1e-5)}
SCORE_RTOL = 1e-5


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msa.load_library()  # raises if the HIP library is missing: no silent fallback


def dev_tensor(store: np.ndarray, device="cuda"):
    """device tensor of a numpy storage array (float32 -> float32, uint16 -> bfloat16)"""
    if store.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(store).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(store)).to(device)


def host_store(t) -> np.ndarray:
    """numpy storage array of a device tensor (bfloat16 -> uint16 bits)"""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def host_f64(t) -> np.ndarray:
    s = host_store(t)
    return (bf16_bits_to_f32(s) if s.dtype == np.uint16 else s).astype(np.float64)


@dataclasses.dataclass
class Dev:
    case: DecodeCase
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    table: torch.Tensor
    lens: torch.Tensor
    S: torch.Tensor
    cfg: object
    cache: object


def to_device(case: DecodeCase, build=True) -> Dev:
    if isinstance(case.q, torch.Tensor):
        q, k, v = case.q, case.k_pool, case.v_pool
    else:
        q = dev_tensor(storage(case.q, case.dtype))
        k = dev_tensor(storage(case.k_pool, case.dtype))
        v = dev_tensor(storage(case.v_pool, case.dtype))
    table = torch.from_numpy(np.ascontiguousarray(case.block_table)).cuda()
    lens = torch.from_numpy(np.ascontiguousarray(case.seq_lens)).cuda()
    S = torch.full((case.num_pages, case.Hkv, case.D), float("nan"), dtype=torch.float32, device="cuda")
    cfg = msa.make_config(case.Hq, case.Hkv, case.top_k, dtype=case.dtype, softmax_scale=case.scale)
    cache = msa.KVCache(k, v, S, table, lens)
    d = Dev(case, q, k, v, table, lens, S, cfg, cache)
    if build:
        msa.msa_build_summaries(cfg, cache, case.B, case.max_seq_len)
    return d


def oracle_inputs(d: Dev) -> dict:
    c = d.case
    return dict(q=host_store(d.q), k_pool=host_store(d.k), v_pool=host_store(d.v),
                block_table=c.block_table, seq_lens=c.seq_lens, Hq=c.Hq, Hkv=c.Hkv, top_k=c.top_k,
                scale=c.scale, P=c.P, keep_sink=int(d.cfg.keep_sink), keep_local=int(d.cfg.keep_local))


def run_decode(d: Dev, max_len=None, k_new=None, v_new=None):
    c = d.case
    max_len = c.max_seq_len if max_len is None else max_len
    mb = (max_len + 63) // 64
    out = torch.empty_like(d.q)
    lse = torch.empty((c.B, c.Hq), dtype=torch.float32, device="cuda")
    idx = torch.empty((c.B, c.Hkv, c.top_k), dtype=torch.int32, device="cuda")
    scores = torch.full((c.B, c.Hkv, max(mb, 1)), float("nan"), dtype=torch.float32, device="cuda")   # every entry written
    msa.msa_decode_step(d.cfg, d.q, d.cache, c.B, max_len, out, k_new=k_new, v_new=v_new, idx_out=idx,
                        scores_out=scores, lse_out=lse)
    torch.cuda.synchronize()
    return dict(o=out, lse=lse, idx=idx, scores=scores[:, :, :mb])


def index_query_abs_bound(q64: np.ndarray, S64: np.ndarray, Hkv: int) -> np.ndarray:
    """sum_d |q_idx,d * S_j,d| per (b, g, j): the scale of each score's summands."""
    B, Hq, D = q64.shape
    G = Hq // Hkv
    qidx = q64.reshape(B, Hkv, G, D).mean(axis=2)                    # [B][Hkv][D]
    return np.einsum("bgd,bjgd->bgj", np.abs(qidx), np.abs(S64))      # [B][Hkv][mb]


def check_scores(gpu_scores: np.ndarray, ref_scores: np.ndarray, bound: np.ndarray, nb: np.ndarray):
    """C16-style comparison of stage-1 scores on the candidate blocks; -inf elsewhere."""
    worst = 0.0
    for b in range(ref_scores.shape[0]):
        n = int(nb[b])
        g_s, r_s = gpu_scores[b, :, :n], ref_scores[b, :, :n]
        tol = SCORE_RTOL * np.maximum(np.abs(r_s), bound[b, :, :n])
        err = np.abs(g_s.astype(np.float64) - r_s)
        assert np.all(err <= tol), "score mismatch b=%d max err/tol=%g" % (b, float((err / tol).max()))
        if n:
            worst = max(worst, float((err / tol).max()))
        assert np.all(np.isneginf(gpu_scores[b, :, n:]))
    return worst


def bf16_step(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at x (8 significant bits): 2^(floor(log2 |x|) - 7); zero at 0."""
    x = np.asarray(x, np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    out[nz] = np.ldexp(1.0, (np.floor(np.log2(np.abs(x[nz]))) - 7).astype(int))
    return out


def check_band(chosen, r, keff, bound_max, keep_sink=0, keep_local=0, where="", slack=0.0):
    """R17 band rule on one row: the forced blocks (if any) are all chosen; among the other
    candidates, blocks clearly above the threshold of the remaining k_eff - |F| slots are in and
    blocks clearly below it are out. `slack` widens the band by a known bound on how far the
    GPU's scores may sit from the oracle's for another reason (bf16 summary rounding)."""
    n = len(r)
    j = np.arange(n)
    forced = (j < keep_sink) | (j >= n - keep_local)
    assert set(j[forced]) <= set(chosen), "forced block missing " + where
    rest = r[~forced]
    kr = keff - int(forced.sum())
    if kr <= 0:
        return
    tau = np.sort(rest)[::-1][kr - 1]
    if np.isneginf(tau):   # fewer finite candidates than slots: every finite one must be kept
        must, never = j[~forced][np.isfinite(rest)], np.zeros(0, np.int64)
    else:
        w = SCORE_RTOL * max(abs(tau), bound_max) + slack
        must = j[~forced][rest > tau + w]
        never = j[~forced][rest < tau - w]
    assert set(must) <= set(chosen), "band: a clearly-in block is missing " + where
    assert not (set(never) & set(chosen)), "band: a clearly-out block was selected " + where


def check_index_sets(gpu_idx, gpu_scores, ref_scores, bound, nb, k, keep_sink=0, keep_local=0, slack=None):
    """Exact same-precision selection plus the band rule against the fp64 scores.
    Returns a boolean array [B][Hkv]: True where the GPU set equals the oracle's."""
    B, Hkv, _ = gpu_idx.shape
    same = np.zeros((B, Hkv), bool)
    for b in range(B):
        n = int(nb[b])
        keff = min(k, n)
        for g in range(Hkv):
            sel = gpu_idx[b, g]
            np.testing.assert_array_equal(sel, oracle.topk(gpu_scores[b, g, :n].astype(np.float64), k,
                                                           keep_sink=keep_sink, keep_local=keep_local))
            chosen = sel[:keff]
            assert np.all(sel[keff:] == -1)
            assert np.all(np.diff(chosen) > 0)
            if keff == 0:
                same[b, g] = True
                continue
            r = ref_scores[b, g, :n]
            check_band(chosen, r, keff, float(bound[b, g, :n].max()), keep_sink, keep_local, "(b=%d g=%d)" % (b, g),
                       0.0 if slack is None else float(slack[b, g]))
            same[b, g] = np.array_equal(chosen, oracle.topk(r, k, keep_sink=keep_sink, keep_local=keep_local)[:keff])
    return same


def assert_close(gpu, ref, dtype, what, lse=False):
    atol, rtol = (LSE_TOL if lse else OUT_TOL)[dtype]
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(gpu)), what + ": non-finite pattern differs"
    err = np.abs(gpu[fin] - ref[fin])
    tol = atol + rtol * np.abs(ref[fin])
    assert np.all(err <= tol), "%s: max err %g (worst err/tol %g)" % (what, float(err.max()), float((err / tol).max()))
    assert np.array_equal(gpu[~fin], ref[~fin]), what + ": non-finite values differ"


def full_decode_check(d: Dev, res: dict, S64=None):
    """End-to-end comparison of one decode step with the oracle; returns the number of
    (b, g) rows whose index set differed from the oracle's inside the band."""
    c = d.case
    inputs = oracle_inputs(d)
    ref = oracle.decode(**inputs)
    if S64 is None:
        S64 = oracle.summaries(k_pool=inputs["k_pool"], block_table=c.block_table, seq_lens=c.seq_lens,
                               Hkv=c.Hkv, D=c.D, P=c.P)
    nb = (c.seq_lens.astype(np.int64) + 63) // 64
    mb = res["scores"].shape[2]
    q64 = host_f64(d.q)
    bound = index_query_abs_bound(q64, S64[:, :mb], c.Hkv)
    gpu_scores = res["scores"].cpu().numpy()
    check_scores(gpu_scores, ref["scores"][:, :, :mb], bound, nb)
    gpu_idx = res["idx"].cpu().numpy()
    same = check_index_sets(gpu_idx, gpu_scores, ref["scores"], bound, nb, c.top_k, inputs["keep_sink"],
                            inputs["keep_local"])
    if not same.all():
        ref = oracle.decode(idx_in=gpu_idx, **inputs)   # stage 2 on the GPU's own selection
    assert_close(host_f64(res["o"]), ref["o"], c.dtype, "o")
    assert_close(res["lse"].cpu().numpy(), ref["lse"], c.dtype, "lse", lse=True)
    return int((~same).sum())
