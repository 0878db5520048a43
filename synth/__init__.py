"""Seeded synthetic inputs for two-stage GQA block-sparse attention.

This module only draws inputs. It computes no step of the attention method:
it draws q, K and V from N(0, 1), rounds them to bf16 when asked, lays K/V out
in 64-token pages (in order or in a seeded permutation) and plants
high-affinity blocks by shifting their keys along a query direction.

Both sides of every check draw from here: the CPU oracle's tests and the HIP
path's tests and benchmark. Nothing here imports either side.

Layouts (row-major):
  q            [B][Hq][D]               decode queries
  k_pool/v_pool[num_pages][Hkv][P][D]   paged cache; page = P tokens of one KV head set
  block_table  [B][max_blocks] int32    logical block j of sequence b -> page id (-1 = unused)
  seq_lens     [B] int32                visible tokens of each sequence
Slots of a page past a sequence's length hold PAD_VALUE, a large finite number,
so that a path which wrongly reads them gives visibly wrong results.

Two generators give the same recipe:
  * numpy (PCG64 streams keyed by (seed, label, tensor, ...)) for CPU-sized cases;
  * torch on a device (torch.Generator seeded from the same keys) for cases whose
    KV cache runs to gigabytes.
Page permutations, planted block positions and sequence lengths are always
drawn with numpy, so both generators agree on the structure for a seed.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

P_DEFAULT = 64
D_DEFAULT = 128
PAD_VALUE = 1000.0  # exactly representable in bf16 (0x447A)

# tensor ids for the per-tensor random streams
_T_Q, _T_K, _T_V, _T_PLANT, _T_PERM, _T_LEN, _T_KNEW, _T_VNEW, _T_QIDX, _T_KIDX, _T_PTOK = range(11)


def rng(seed: int, *stream: int) -> np.random.Generator:
    """An independent PCG64 stream keyed by (seed, *stream)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, stream)])))


def _torch_seed(seed: int, *stream: int) -> int:
    return int(np.random.SeedSequence([int(seed), *map(int, stream)]).generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


# ---------------------------------------------------------------------------
# bf16 storage helpers (round-to-nearest-even, as IEEE conversion does)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array whose values are the bf16 roundings of x."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def loguniform_lengths(B: int, lo: int, hi: int, cap: int, seed: int, label: int = 4) -> np.ndarray:
    """B integer lengths floor(exp(U(ln lo, ln hi))), clipped to [lo, hi];
    the whole batch is redrawn from the next sub-stream while the sum exceeds cap."""
    attempt = 0
    while True:
        r = rng(seed, label, _T_LEN, attempt)
        x = np.floor(np.exp(r.uniform(math.log(lo), math.log(hi), size=B))).astype(np.int64)
        x = np.clip(x, lo, hi)
        if int(x.sum()) <= cap:
            return x.astype(np.int32)
        attempt += 1


# ---------------------------------------------------------------------------
# Case containers
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class DecodeCase:
    dtype: str                 # "f32" or "bf16": storage type of q, K, V (and of the output)
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    top_k: int
    scale: float
    seq_lens: np.ndarray       # [B] int32
    block_table: np.ndarray    # [B][max_blocks] int32
    num_pages: int
    q: object                  # [B][Hq][D]: float32 numpy array (values exact in dtype) or torch tensor
    k_pool: object             # [num_pages][Hkv][P][D]
    v_pool: object
    planted: Dict[Tuple[int, int], List[int]]  # (b, g) -> planted logical blocks
    label: int = 0
    seed: int = 0

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.B else 0


@dataclasses.dataclass
class PrefillCase:
    dtype: str
    Hq: int
    Hkv: int
    D: int
    P: int
    top_k: int
    scale: float
    past_len: int
    T: int
    block_table: np.ndarray    # [1][max_blocks] int32, covers past_len + T tokens
    num_pages: int
    q: object                  # [T][Hq][D]
    k_new: object              # [T][Hkv][D]
    v_new: object
    k_pool: object             # [num_pages][Hkv][P][D]; pages of the new chunk hold PAD_VALUE
    v_pool: object
    planted: Dict[Tuple[int, int], int]  # (tile, g) -> planted cached block
    label: int = 0
    seed: int = 0

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


@dataclasses.dataclass
class IndexCase:
    """Inputs of the index branch: one index query per (sequence, group) and one single-head
    index key per cached token, paged like K."""
    dtype: str
    B: int
    Hkv: int
    Di: int
    P: int
    top_k: int
    seq_lens: np.ndarray       # [B] int32
    block_table: np.ndarray    # [B][max_blocks] int32
    num_pages: int
    q_idx: object              # [B][Hkv][Di]
    index_keys: object         # [num_pages][P][Di]
    planted: Dict[Tuple[int, int], List[int]]  # (b, g) -> logical blocks holding a planted token
    label: int = 0
    seed: int = 0

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.B else 0


def storage(x, dtype: str):
    """numpy storage view of a float32 numpy array: itself (f32) or its bf16 bit patterns."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x)


# ---------------------------------------------------------------------------
# Shared structure: pages, permutation, planted positions
# ---------------------------------------------------------------------------
def _layout(lens: Sequence[int], P: int, permute: bool, seed: int, label: int):
    lens = np.asarray(lens, dtype=np.int64)
    nb = (lens + P - 1) // P
    num_pages = int(nb.sum())
    order = np.arange(num_pages, dtype=np.int64)
    if permute and num_pages > 1:
        order = rng(seed, label, _T_PERM).permutation(num_pages)
    max_blocks = int(max(1, nb.max() if len(nb) else 1))
    table = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nb):
        table[b, :n] = order[off:off + n]
        off += int(n)
    return nb, num_pages, table


def _plant_positions(nb: np.ndarray, Hkv: int, plant, seed: int, label: int):
    """(b, g) -> sorted list of distinct logical blocks to plant."""
    kind, amount = plant if plant is not None else ("count", 0)
    out = {}
    for b, n in enumerate(nb):
        n = int(n)
        for g in range(Hkv):
            if kind == "count":
                c = int(amount)
            elif kind == "frac":
                c = max(1, int(round(amount * n)))
            else:
                raise ValueError(kind)
            c = min(c, n)
            r = rng(seed, label, _T_PLANT, b, g)
            out[(b, g)] = sorted(int(j) for j in r.choice(n, size=c, replace=False)) if c else []
    return out


def _unit(v: np.ndarray) -> np.ndarray:
    v = v.astype(np.float64)
    n = np.linalg.norm(v)
    return (v / n).astype(np.float32) if n > 0 else np.zeros_like(v, dtype=np.float32)


# ---------------------------------------------------------------------------
# numpy generator (CPU-sized cases)
# ---------------------------------------------------------------------------
def make_decode_case(*, B: int = 1, Hq: int, Hkv: int, lens: Sequence[int], top_k: int,
                     dtype: str = "bf16", seed: int = 0, label: int = 0,
                     plant=("count", 3), permute: bool = False, D: int = D_DEFAULT,
                     P: int = P_DEFAULT, scale: Optional[float] = None,
                     plant_shift: float = 0.5) -> DecodeCase:
    """Decode inputs with numpy: q, K, V ~ N(0,1); planted blocks get +plant_shift*u
    on their valid keys, u = unit vector along the sum of the group's query heads."""
    assert len(lens) == B and Hq % Hkv == 0
    G = Hq // Hkv
    nb, num_pages, table = _layout(lens, P, permute, seed, label)
    rnd = (lambda a: a) if dtype == "f32" else round_to_bf16
    q = rnd(rng(seed, label, _T_Q).standard_normal((B, Hq, D), dtype=np.float32))
    k = rng(seed, label, _T_K).standard_normal((num_pages, Hkv, P, D), dtype=np.float32)
    v = rng(seed, label, _T_V).standard_normal((num_pages, Hkv, P, D), dtype=np.float32)
    planted = _plant_positions(nb, Hkv, plant, seed, label)
    for (b, g), blocks in planted.items():
        u = _unit(q[b, g * G:(g + 1) * G].sum(axis=0))
        for j in blocks:
            n_j = min(P, int(lens[b]) - j * P)
            k[table[b, j], g, :n_j, :] += plant_shift * u
    k, v = rnd(k), rnd(v)
    for b in range(B):
        n = int(lens[b])
        if n > 0 and n % P:
            last = table[b, (n - 1) // P]
            k[last, :, n % P:, :] = PAD_VALUE
            v[last, :, n % P:, :] = PAD_VALUE
    return DecodeCase(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, P=P, top_k=top_k,
                      scale=(1.0 / math.sqrt(D)) if scale is None else scale,
                      seq_lens=np.asarray(lens, dtype=np.int32), block_table=table,
                      num_pages=num_pages, q=q, k_pool=k, v_pool=v, planted=planted,
                      label=label, seed=seed)


def make_prefill_case(*, Hq: int, Hkv: int, past_len: int, T: int, top_k: int,
                      dtype: str = "bf16", seed: int = 0, label: int = 3,
                      permute: bool = False, plant: bool = True, D: int = D_DEFAULT,
                      P: int = P_DEFAULT, scale: Optional[float] = None,
                      plant_shift: float = 0.5) -> PrefillCase:
    """Prefill-chunk inputs with numpy. The cache holds past_len tokens; T new tokens
    (q, k_new, v_new) follow. One cached block per (tile, group) is planted along that
    tile's query direction (sum over the tile's tokens and the group's heads)."""
    assert past_len % P == 0 and Hq % Hkv == 0
    G = Hq // Hkv
    total = past_len + T
    nb, num_pages, table = _layout([total], P, permute, seed, label)
    past_blocks = past_len // P
    rnd = (lambda a: a) if dtype == "f32" else round_to_bf16
    q = rnd(rng(seed, label, _T_Q).standard_normal((T, Hq, D), dtype=np.float32))
    k_new = rnd(rng(seed, label, _T_KNEW).standard_normal((T, Hkv, D), dtype=np.float32))
    v_new = rnd(rng(seed, label, _T_VNEW).standard_normal((T, Hkv, D), dtype=np.float32))
    k = rng(seed, label, _T_K).standard_normal((num_pages, Hkv, P, D), dtype=np.float32)
    v = rng(seed, label, _T_V).standard_normal((num_pages, Hkv, P, D), dtype=np.float32)
    ntiles = (T + P - 1) // P
    planted = {}
    if plant and past_blocks > 0:
        for g in range(Hkv):
            r = rng(seed, label, _T_PLANT, 0, g)
            blocks = r.choice(past_blocks, size=ntiles, replace=ntiles > past_blocks)
            for tau in range(ntiles):
                rows = q[tau * P:min(T, (tau + 1) * P), g * G:(g + 1) * G]
                u = _unit(rows.reshape(-1, D).sum(axis=0))
                j = int(blocks[tau])
                k[table[0, j], g, :, :] += plant_shift * u
                planted[(tau, g)] = j
    k, v = rnd(k), rnd(v)
    for j in range(past_blocks, int(nb[0])):
        k[table[0, j]] = PAD_VALUE
        v[table[0, j]] = PAD_VALUE
    return PrefillCase(dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, P=P, top_k=top_k,
                       scale=(1.0 / math.sqrt(D)) if scale is None else scale,
                       past_len=past_len, T=T, block_table=table, num_pages=num_pages,
                       q=q, k_new=k_new, v_new=v_new, k_pool=k, v_pool=v,
                       planted=planted, label=label, seed=seed)


def _index_plants(q_idx: np.ndarray, lens, nb, table, Hkv: int, P: int, plant, seed: int, label: int,
                  plant_shift: float):
    """page -> [(token slot, shift vector)]: one token of each planted block, drawn among the
    block's valid tokens, is moved by plant_shift along the unit direction of its group's index
    query (a single token, so only a max over tokens is sure to see it)."""
    planted = _plant_positions(nb, Hkv, plant, seed, label)
    by_page: Dict[int, list] = {}
    for (b, g), blocks in planted.items():
        u = plant_shift * _unit(q_idx[b, g])
        for j in blocks:
            n_j = min(P, int(lens[b]) - j * P)
            t = int(rng(seed, label, _T_PTOK, b, g, j).integers(n_j))
            by_page.setdefault(int(table[b, j]), []).append((t, u))
    return planted, by_page


def make_index_case(*, B: int = 1, Hkv: int, lens: Sequence[int], top_k: int, dtype: str = "bf16",
                    seed: int = 0, label: int = 5, plant=("count", 3), permute: bool = False,
                    Di: int = D_DEFAULT, P: int = P_DEFAULT, plant_shift: float = 10.0) -> IndexCase:
    """Index-branch inputs with numpy: q_idx and K_idx ~ N(0,1); planted blocks get one token
    shifted along their group's index query; slots past a sequence's length hold PAD_VALUE."""
    assert len(lens) == B
    nb, num_pages, table = _layout(lens, P, permute, seed, label)
    rnd = (lambda a: a) if dtype == "f32" else round_to_bf16
    q_idx = rnd(rng(seed, label, _T_QIDX).standard_normal((B, Hkv, Di), dtype=np.float32))
    keys = rng(seed, label, _T_KIDX).standard_normal((num_pages, P, Di), dtype=np.float32)
    planted, by_page = _index_plants(q_idx, lens, nb, table, Hkv, P, plant, seed, label, plant_shift)
    for page, items in by_page.items():
        for t, u in items:
            keys[page, t, :] += u
    keys = rnd(keys)
    for b in range(B):
        n = int(lens[b])
        if n > 0 and n % P:
            keys[table[b, (n - 1) // P], n % P:, :] = PAD_VALUE
    return IndexCase(dtype=dtype, B=B, Hkv=Hkv, Di=Di, P=P, top_k=top_k,
                     seq_lens=np.asarray(lens, dtype=np.int32), block_table=table, num_pages=num_pages,
                     q_idx=q_idx, index_keys=keys, planted=planted, label=label, seed=seed)


# ---------------------------------------------------------------------------
# torch-on-device generator (gigabyte caches); same recipe, torch RNG for the bulk draws
# ---------------------------------------------------------------------------
def _torch_normal(shape, seed_key, device, torch):
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(*seed_key))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def make_decode_case_torch(*, B: int = 1, Hq: int, Hkv: int, lens: Sequence[int], top_k: int,
                           dtype: str = "bf16", seed: int = 0, label: int = 0,
                           plant=("count", 3), permute: bool = False, D: int = D_DEFAULT,
                           P: int = P_DEFAULT, scale: Optional[float] = None,
                           device="cuda", plant_shift: float = 0.5,
                           chunk_pages: int = 8192) -> DecodeCase:
    """The recipe of make_decode_case with the bulk draws made by torch on `device`.
    q, k_pool, v_pool are torch tensors (float32 or bfloat16); everything else is numpy."""
    import torch
    assert len(lens) == B and Hq % Hkv == 0
    G = Hq // Hkv
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    nb, num_pages, table = _layout(lens, P, permute, seed, label)
    q32 = _torch_normal((B, Hq, D), (seed, label, _T_Q), device, torch)
    q = q32.to(tdt)
    qf = q.float().cpu().numpy()
    planted = _plant_positions(nb, Hkv, plant, seed, label)
    # page -> list of (g, n_valid, shift vector)
    plant_by_page: Dict[int, list] = {}
    for (b, g), blocks in planted.items():
        u = plant_shift * _unit(qf[b, g * G:(g + 1) * G].sum(axis=0))
        for j in blocks:
            n_j = min(P, int(lens[b]) - j * P)
            plant_by_page.setdefault(int(table[b, j]), []).append((g, n_j, u))
    # last partial page of each sequence -> first padded slot
    pad_at = {}
    for b in range(B):
        n = int(lens[b])
        if n > 0 and n % P:
            pad_at[int(table[b, (n - 1) // P])] = n % P
    k_pool = torch.empty((num_pages, Hkv, P, D), dtype=tdt, device=device)
    v_pool = torch.empty((num_pages, Hkv, P, D), dtype=tdt, device=device)
    for c0 in range(0, num_pages, chunk_pages):
        c1 = min(num_pages, c0 + chunk_pages)
        kc = _torch_normal((c1 - c0, Hkv, P, D), (seed, label, _T_K, c0), device, torch)
        vc = _torch_normal((c1 - c0, Hkv, P, D), (seed, label, _T_V, c0), device, torch)
        for page in range(c0, c1):
            for (g, n_j, u) in plant_by_page.get(page, ()):
                kc[page - c0, g, :n_j, :] += torch.from_numpy(u).to(device)
        for page, s in pad_at.items():
            if c0 <= page < c1:
                kc[page - c0, :, s:, :] = PAD_VALUE
                vc[page - c0, :, s:, :] = PAD_VALUE
        k_pool[c0:c1] = kc.to(tdt)
        v_pool[c0:c1] = vc.to(tdt)
        del kc, vc
    return DecodeCase(dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, P=P, top_k=top_k,
                      scale=(1.0 / math.sqrt(D)) if scale is None else scale,
                      seq_lens=np.asarray(lens, dtype=np.int32), block_table=table,
                      num_pages=num_pages, q=q, k_pool=k_pool, v_pool=v_pool,
                      planted=planted, label=label, seed=seed)


def make_index_case_torch(*, B: int = 1, Hkv: int, lens: Sequence[int], top_k: int, dtype: str = "bf16",
                          seed: int = 0, label: int = 5, plant=("count", 3), permute: bool = False,
                          Di: int = D_DEFAULT, P: int = P_DEFAULT, plant_shift: float = 10.0,
                          device="cuda", chunk_pages: int = 16384) -> IndexCase:
    """The recipe of make_index_case with the bulk draws made by torch on `device`; q_idx and
    index_keys are torch tensors (float32 or bfloat16)."""
    import torch
    assert len(lens) == B
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    nb, num_pages, table = _layout(lens, P, permute, seed, label)
    q_idx = _torch_normal((B, Hkv, Di), (seed, label, _T_QIDX), device, torch).to(tdt)
    planted, by_page = _index_plants(q_idx.float().cpu().numpy(), lens, nb, table, Hkv, P, plant, seed,
                                     label, plant_shift)
    pad_at = {}
    for b in range(B):
        n = int(lens[b])
        if n > 0 and n % P:
            pad_at[int(table[b, (n - 1) // P])] = n % P
    keys = torch.empty((num_pages, P, Di), dtype=tdt, device=device)
    for c0 in range(0, num_pages, chunk_pages):
        c1 = min(num_pages, c0 + chunk_pages)
        kc = _torch_normal((c1 - c0, P, Di), (seed, label, _T_KIDX, c0), device, torch)
        for page in range(c0, c1):
            for t, u in by_page.get(page, ()):
                kc[page - c0, t, :] += torch.from_numpy(u).to(device)
        for page, s in pad_at.items():
            if c0 <= page < c1:
                kc[page - c0, s:, :] = PAD_VALUE
        keys[c0:c1] = kc.to(tdt)
        del kc
    return IndexCase(dtype=dtype, B=B, Hkv=Hkv, Di=Di, P=P, top_k=top_k,
                     seq_lens=np.asarray(lens, dtype=np.int32), block_table=table, num_pages=num_pages,
                     q_idx=q_idx, index_keys=keys, planted=planted, label=label, seed=seed)


def make_prefill_case_torch(*, Hq: int, Hkv: int, past_len: int, T: int, top_k: int,
                            dtype: str = "bf16", seed: int = 0, label: int = 3,
                            permute: bool = False, plant: bool = True, D: int = D_DEFAULT,
                            P: int = P_DEFAULT, scale: Optional[float] = None,
                            device="cuda", plant_shift: float = 0.5) -> PrefillCase:
    """The recipe of make_prefill_case with torch draws on `device`."""
    import torch
    assert past_len % P == 0 and Hq % Hkv == 0
    G = Hq // Hkv
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    total = past_len + T
    nb, num_pages, table = _layout([total], P, permute, seed, label)
    past_blocks = past_len // P
    q = _torch_normal((T, Hq, D), (seed, label, _T_Q), device, torch).to(tdt)
    k_new = _torch_normal((T, Hkv, D), (seed, label, _T_KNEW), device, torch).to(tdt)
    v_new = _torch_normal((T, Hkv, D), (seed, label, _T_VNEW), device, torch).to(tdt)
    k32 = _torch_normal((num_pages, Hkv, P, D), (seed, label, _T_K, 0), device, torch)
    v32 = _torch_normal((num_pages, Hkv, P, D), (seed, label, _T_V, 0), device, torch)
    ntiles = (T + P - 1) // P
    planted = {}
    if plant and past_blocks > 0:
        qf = q.float()
        for g in range(Hkv):
            r = rng(seed, label, _T_PLANT, 0, g)
            blocks = r.choice(past_blocks, size=ntiles, replace=ntiles > past_blocks)
            for tau in range(ntiles):
                rows = qf[tau * P:min(T, (tau + 1) * P), g * G:(g + 1) * G].reshape(-1, D)
                u = _unit(rows.sum(dim=0).cpu().numpy())
                j = int(blocks[tau])
                k32[int(table[0, j]), g] += plant_shift * torch.from_numpy(u).to(device)
                planted[(tau, g)] = j
    new_pages = torch.as_tensor(table[0, past_blocks:int(nb[0])].astype(np.int64), device=device)
    k32[new_pages] = PAD_VALUE
    v32[new_pages] = PAD_VALUE
    k_pool, v_pool = k32.to(tdt), v32.to(tdt)
    del k32, v32
    return PrefillCase(dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, P=P, top_k=top_k,
                       scale=(1.0 / math.sqrt(D)) if scale is None else scale,
                       past_len=past_len, T=T, block_table=table, num_pages=num_pages,
                       q=q, k_new=k_new, v_new=v_new, k_pool=k_pool, v_pool=v_pool,
                       planted=planted, label=label, seed=seed)


# ---------------------------------------------------------------------------
# The five workloads, at full size
# ---------------------------------------------------------------------------
def workload(name: str, seed: int = 0) -> dict:
    """Keyword arguments of the generator for one of the five named workloads."""
    if name == "decode_f32_4k":
        return dict(B=1, Hq=8, Hkv=1, lens=[4096], top_k=16, dtype="f32", seed=seed, label=0,
                    plant=("count", 3), permute=False)
    if name == "decode_bf16_b8_128k":
        return dict(B=8, Hq=32, Hkv=8, lens=[131072] * 8, top_k=32, dtype="bf16", seed=seed,
                    label=1, plant=("frac", 0.01), permute=False)
    if name == "decode_bf16_1m_paged":
        return dict(B=1, Hq=32, Hkv=8, lens=[1048576], top_k=64, dtype="bf16", seed=seed,
                    label=2, plant=("count", 16), permute=True)
    if name == "prefill_bf16_4k_on_256k":
        return dict(Hq=32, Hkv=8, past_len=262144, T=4096, top_k=32, dtype="bf16", seed=seed,
                    label=3, permute=False, plant=True)
    if name == "decode_bf16_mixed_b32":
        lens = loguniform_lengths(32, 4096, 1048576, 8388608, seed, label=4)
        return dict(B=32, Hq=32, Hkv=8, lens=[int(x) for x in lens], top_k=64, dtype="bf16",
                    seed=seed, label=4, plant=("frac", 0.01), permute=True)
    raise KeyError(name)


WORKLOADS = ("decode_f32_4k", "decode_bf16_b8_128k", "decode_bf16_1m_paged",
             "prefill_bf16_4k_on_256k", "decode_bf16_mixed_b32")
