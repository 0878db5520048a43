"""Test-side helpers: logical views of paged inputs and library reference routines.

Nothing here reimplements the oracle: dense attention comes from torch's
scaled_dot_product_attention / logsumexp in float64 on the CPU.
"""
from __future__ import annotations

import numpy as np
import torch

from synth import bf16_bits_to_f32


def as_f64(store: np.ndarray) -> np.ndarray:
    """float64 values of a storage array (float32 or bf16 bit patterns)."""
    if store.dtype == np.uint16:
        return bf16_bits_to_f32(store).astype(np.float64)
    return np.asarray(store, dtype=np.float64)


def logical_kv(pool: np.ndarray, table: np.ndarray, b: int, N: int) -> np.ndarray:
    """[N][Hkv][D] view of sequence b's first N tokens in a [pages][Hkv][P][D] pool."""
    P = pool.shape[2]
    t = np.arange(N)
    pages = table[b, t // P]
    return pool[pages, :, t % P, :]


def dense_gqa(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, mask=None):
    """Dense GQA attention with torch SDPA (float64, CPU).
    q [Hq][D] or [T][Hq][D]; K, V [N][Hkv][D]; mask [.., N] bool (True = visible).
    Returns (o, lse) with o shaped like q and lse [Hq] or [T][Hq]."""
    single = q.ndim == 2
    qq = torch.from_numpy(np.asarray(q, np.float64))
    if single:
        qq = qq[None]
    T, Hq, D = qq.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    Kt = torch.from_numpy(np.asarray(K, np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
    Vt = torch.from_numpy(np.asarray(V, np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
    Q = qq.permute(1, 0, 2)  # [Hq][T][D]
    m = None
    if mask is not None:
        mm = torch.from_numpy(np.asarray(mask, bool))
        if mm.ndim == 1:
            mm = mm[None]
        m = mm[None].expand(Hq, T, -1)
    o = torch.nn.functional.scaled_dot_product_attention(Q[None], Kt[None], Vt[None],
                                                         attn_mask=None if m is None else m[None],
                                                         scale=scale)[0]
    logits = torch.matmul(Q, Kt.transpose(1, 2)) * scale
    if m is not None:
        logits = logits.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)  # [Hq][T]
    o = o.permute(1, 0, 2).numpy()
    lse = lse.permute(1, 0).numpy()
    if single:
        return o[0], lse[0]
    return o, lse


def decode_inputs(case) -> dict:
    """Oracle keyword arguments for a numpy DecodeCase."""
    from synth import storage
    return dict(q=storage(case.q, case.dtype), k_pool=storage(case.k_pool, case.dtype),
                v_pool=storage(case.v_pool, case.dtype), block_table=case.block_table,
                seq_lens=case.seq_lens, Hq=case.Hq, Hkv=case.Hkv, top_k=case.top_k,
                scale=case.scale, P=case.P)


def prefill_inputs(case) -> dict:
    from synth import storage
    return dict(q=storage(case.q, case.dtype), k_new=storage(case.k_new, case.dtype),
                v_new=storage(case.v_new, case.dtype), k_pool=storage(case.k_pool, case.dtype),
                v_pool=storage(case.v_pool, case.dtype), block_table=case.block_table,
                past_len=case.past_len, Hq=case.Hq, Hkv=case.Hkv, top_k=case.top_k,
                scale=case.scale, P=case.P)
