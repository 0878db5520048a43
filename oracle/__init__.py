"""CPU oracle for two-stage GQA block-sparse attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package. It wraps `oracle.c` (plain fp64 C, built with gcc into `liboracle.so` next to this
file) with ctypes. It shares no code with the HIP library and never imports it.

What the oracle computes, and the readings taken where the source page is silent, are
stated in the header of oracle.c ("MiniMax goes sparse: decoding M3's attention from a
single diagram", §1 Step 1 and Step 2).

Inputs are numpy arrays in storage form: float32, or uint16 bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# a test may point the wrapper at another build of oracle.c (the mutation test does)
_LIB_OVERRIDE = os.environ.get("MSA_ORACLE_LIB")

F32, BF16 = 0, 1
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (atomically replaced)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not _LIB_OVERRIDE and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(path)
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.orc_topk.argtypes = [P, I, I, P]
        lib.orc_topk.restype = I
        lib.orc_topk_forced.argtypes = [P, I, I, I, I, P]
        lib.orc_topk_forced.restype = I
        lib.orc_decode.argtypes = [I, I, I, I, I, I, I, I, I, D, I, P, P, P, I, P, I, P, P, P, P, P, P, P, P, I]
        lib.orc_decode.restype = I
        lib.orc_summaries.argtypes = [I, I, I, I, I, I, P, I, P, I, P, P]
        lib.orc_summaries.restype = I
        lib.orc_prefill.argtypes = [I, I, I, I, I, I, I, I, D, I, P, P, P, P, P, I, P, I, I, I, I, I, P, P, P, P, P, I]
        lib.orc_select_index.argtypes = [I, I, I, I, I, I, I, I, P, P, I, P, I, P, P, P]
        lib.orc_select_index.restype = I
        lib.orc_prefill.restype = I
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _c(a, dt=None):
    return np.ascontiguousarray(a if dt is None else np.asarray(a, dtype=dt))


def _summary_flag(summary_dtype: str) -> int:
    return {"f32": 0, "bf16": 1}[summary_dtype]


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count() or 1)


def topk(scores: np.ndarray, k: int, keep_sink: int = 0, keep_local: int = 0) -> np.ndarray:
    """k_eff = min(k, n) block indices by (score desc, index asc), ascending, padded with -1.
    keep_sink / keep_local (reading R9): the first / last blocks that are always kept."""
    s = _c(scores, np.float64)
    out = np.empty(k, dtype=np.int32)
    if keep_sink or keep_local:
        rc = _load().orc_topk_forced(_ptr(s), int(s.shape[0]), int(k), int(keep_sink), int(keep_local), _ptr(out))
    else:
        rc = _load().orc_topk(_ptr(s), int(s.shape[0]), int(k), _ptr(out))
    if rc < 0:
        raise RuntimeError("orc_topk failed")
    return out


def summaries(*, k_pool, block_table, seq_lens, Hkv: int, D: int, P: int, summary_dtype: str = "f32") -> np.ndarray:
    """Block summaries [B][max_blocks][Hkv][D] (fp64), zero past each sequence's blocks;
    summary_dtype "bf16" rounds each one to bf16 (reading R10)."""
    k_pool = _c(k_pool)
    table = _c(block_table, np.int32)
    lens = _c(seq_lens, np.int32)
    B, mb = table.shape
    out = np.empty((B, mb, Hkv, D), dtype=np.float64)
    rc = _load().orc_summaries(B, Hkv, D, P, _dtype_code(k_pool), _summary_flag(summary_dtype), _ptr(k_pool),
                               int(k_pool.shape[0]), _ptr(table), mb, _ptr(lens), _ptr(out))
    if rc != 0:
        raise RuntimeError("orc_summaries failed (%d)" % rc)
    return out


def select_index(*, q_idx, index_keys, block_table, seq_lens, top_k: int, P: int = 64, keep_sink: int = 0,
                 keep_local: int = 0) -> dict:
    """The index branch of [MGS §1 Step 1] (reading R8): token scores of each group's index query
    against the single-head index keys, Block Max Pool, TopK. q_idx [B][Hkv][Di] and
    index_keys [num_pages][P][Di] share one storage dtype (float32, or bf16 bits as uint16).
    Returns scores [B][Hkv][max_blocks] (fp64, -inf past the blocks) and idx [B][Hkv][top_k]."""
    qi = _c(q_idx)
    ik = _c(index_keys)
    if _dtype_code(qi) != _dtype_code(ik):
        raise ValueError("q_idx and index_keys must share a dtype")
    table = _c(block_table, np.int32)
    lens = _c(seq_lens, np.int32)
    B, Hkv, Di = qi.shape
    mb = table.shape[1]
    scores = np.empty((B, Hkv, mb), dtype=np.float64)
    idx = np.empty((B, Hkv, top_k), dtype=np.int32)
    rc = _load().orc_select_index(B, Hkv, Di, P, top_k, int(keep_sink), int(keep_local), _dtype_code(qi), _ptr(qi), _ptr(ik), int(ik.shape[0]),
                                  _ptr(table), mb, _ptr(lens), _ptr(scores), _ptr(idx))
    if rc != 0:
        raise RuntimeError("orc_select_index failed (%d)" % rc)
    return {"scores": scores, "idx": idx}


def decode(*, q, k_pool, v_pool, block_table, seq_lens, Hq: int, Hkv: int, top_k: int,
           scale: float, P: int = 64, summaries_in: Optional[np.ndarray] = None,
           idx_in: Optional[np.ndarray] = None, want_weights: bool = False,
           nthreads: Optional[int] = None, keep_sink: int = 0, keep_local: int = 0,
           summary_dtype: str = "f32") -> dict:
    """Decode step over B sequences. Returns scores [B][Hkv][max_blocks], idx [B][Hkv][top_k],
    o [B][Hq][D], lse [B][Hq] (fp64) and, if asked, w [B][Hq][top_k*P]."""
    q, k_pool, v_pool = _c(q), _c(k_pool), _c(v_pool)
    dt = _dtype_code(q)
    assert _dtype_code(k_pool) == dt and _dtype_code(v_pool) == dt
    table = _c(block_table, np.int32)
    lens = _c(seq_lens, np.int32)
    B, mb = table.shape
    D = q.shape[-1]
    scores = np.empty((B, Hkv, mb), dtype=np.float64)
    idx = np.empty((B, Hkv, top_k), dtype=np.int32)
    o = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    w = np.empty((B, Hq, top_k * P), dtype=np.float64) if want_weights else None
    s_in = None if summaries_in is None else _c(summaries_in, np.float64)
    i_in = None if idx_in is None else _c(idx_in, np.int32)
    rc = _load().orc_decode(B, Hq, Hkv, D, P, top_k, int(keep_sink), int(keep_local), _summary_flag(summary_dtype),
                            float(scale), dt, _ptr(q), _ptr(k_pool),
                            _ptr(v_pool), int(k_pool.shape[0]), _ptr(table), mb, _ptr(lens),
                            _ptr(s_in), _ptr(i_in), _ptr(scores), _ptr(idx), _ptr(o), _ptr(lse),
                            _ptr(w), int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("orc_decode failed (%d)" % rc)
    out = dict(scores=scores, idx=idx, o=o, lse=lse)
    if want_weights:
        out["w"] = w
    return out


def prefill(*, q, k_new, v_new, k_pool, v_pool, block_table, past_len: int, Hq: int, Hkv: int,
            top_k: int, scale: float, P: int = 64, tiles: Optional[tuple] = None,
            idx_in: Optional[np.ndarray] = None, nthreads: Optional[int] = None, keep_sink: int = 0,
            keep_local: int = 0, summary_dtype: str = "f32") -> dict:
    """Prefill chunk of T tokens on one sequence. Returns scores [ntiles][Hkv][max_blocks],
    idx [ntiles][Hkv][top_k+1], o [T][Hq][D], lse [T][Hq]; only tiles [lo, hi) are computed
    (rows of other tiles are NaN). idx_in ([ntiles][Hkv][top_k+1]) replaces the selection."""
    q, k_new, v_new, k_pool, v_pool = map(_c, (q, k_new, v_new, k_pool, v_pool))
    dt = _dtype_code(q)
    table = _c(block_table, np.int32).reshape(-1)
    T, _, D = q.shape
    ntiles = (T + P - 1) // P
    lo, hi = tiles if tiles is not None else (0, ntiles)
    mb = table.shape[0]
    scores = np.full((ntiles, Hkv, mb), np.nan)
    idx = np.full((ntiles, Hkv, top_k + 1), -2, dtype=np.int32)
    o = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    rc = _load().orc_prefill(Hq, Hkv, D, P, top_k, int(keep_sink), int(keep_local), _summary_flag(summary_dtype),
                             float(scale), dt, _ptr(q), _ptr(k_new),
                             _ptr(v_new), _ptr(k_pool), _ptr(v_pool), int(k_pool.shape[0]),
                             _ptr(table), mb, int(past_len), int(T), int(lo), int(hi),
                             _ptr(None if idx_in is None else _c(idx_in, np.int32)),
                             _ptr(scores), _ptr(idx), _ptr(o), _ptr(lse),
                             int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError("orc_prefill failed (%d)" % rc)
    return dict(scores=scores, idx=idx, o=o, lse=lse)
