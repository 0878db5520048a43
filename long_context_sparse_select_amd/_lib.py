"""ctypes binding of libmsa.so. See include/msa.h for the contract of every call."""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP = range(5)
MSA_F32, MSA_BF16 = 0, 1
MSA_SCORE_MEAN_KEY, MSA_SCORE_MAX_TOKEN = 0, 1
MSA_OP_SELECT, MSA_OP_ATTEND, MSA_OP_DECODE, MSA_OP_PREFILL = range(4)

EXPORTED = ("msa_workspace_size", "msa_build_summaries", "msa_score", "msa_select", "msa_select_index",
            "msa_attend", "msa_decode_step", "msa_decode_step_noalloc", "msa_prefill_chunk", "msa_prefill_attend",
            "msa_status_string")
# measurement probes of the GPU itself (include/msa_probe.h)
EXPORTED_PROBES = ("msa_probe_hbm_read", "msa_probe_mfma_bf16")


class MsaConfig(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("score_mode", ctypes.c_int32),
                ("keep_local", ctypes.c_int32), ("q_tile", ctypes.c_int32),
                ("keep_sink", ctypes.c_int32), ("summary_dtype", ctypes.c_int32)]


class MsaKvCache(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("summaries", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("num_pages", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32)]


class MsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s" % (where, msa_status_string(status)))
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmsa.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libmsa.so is not built (%s); run `python __graft_entry__.py` or "
                               "long_context_sparse_select_amd/build.py" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        V, I, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        C, K = ctypes.POINTER(MsaConfig), ctypes.POINTER(MsaKvCache)
        lib.msa_workspace_size.argtypes = [C, I, I, I, I, ctypes.POINTER(Z)]
        lib.msa_build_summaries.argtypes = [C, K, I, I, V]
        lib.msa_score.argtypes = [C, V, K, I, I, V, V]
        lib.msa_select.argtypes = [C, V, K, I, I, V, V, V, Z, V]
        lib.msa_select_index.argtypes = [C, V, V, I, K, I, I, V, V, V, Z, V]
        lib.msa_attend.argtypes = [C, V, K, I, I, V, V, V, V, Z, V]
        lib.msa_decode_step.argtypes = [C, V, K, I, I, V, V, V, V, V, V, V, Z, V]
        lib.msa_prefill_chunk.argtypes = [C, V, V, V, K, I, I, V, V, V, V, V, Z, V]
        lib.msa_prefill_attend.argtypes = [C, V, K, I, I, V, V, V, V]
        lib.msa_decode_step_noalloc.argtypes = [C, V, K, I, I, V, V, V, V, V, V, V]
        for name in EXPORTED[:-1]:
            getattr(lib, name).restype = ctypes.c_int
        lib.msa_status_string.argtypes = [ctypes.c_int]
        lib.msa_status_string.restype = ctypes.c_char_p
        lib.msa_probe_hbm_read.argtypes = [V, Z, V, V]
        lib.msa_probe_mfma_bf16.argtypes = [V, I, I, V]
        for name in EXPORTED_PROBES:
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def msa_status_string(status: int) -> str:
    return load_library().msa_status_string(int(status)).decode()


def make_config(num_q_heads: int, num_kv_heads: int, top_k: int, dtype: str = "bf16",
                softmax_scale: Optional[float] = None, head_dim: int = 128, block_size: int = 64,
                score_mode: int = MSA_SCORE_MEAN_KEY, keep_local: int = 0,
                q_tile: int = 64, keep_sink: int = 0, summary_dtype: str = "f32") -> MsaConfig:
    dt = {"f32": MSA_F32, "bf16": MSA_BF16}[dtype]
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else softmax_scale
    return MsaConfig(num_q_heads, num_kv_heads, head_dim, block_size, top_k, scale, dt, dt, dt,
                     score_mode, keep_local, q_tile, keep_sink, {"f32": MSA_F32, "bf16": MSA_BF16}[summary_dtype])


@dataclasses.dataclass
class KVCache:
    """Device tensors of a paged cache (see msa.h for layouts)."""
    k_pages: object       # [num_pages][Hkv][64][128]
    v_pages: object
    summaries: object     # [num_pages][Hkv][128] float32 or bfloat16 (the config's summary_dtype)
    block_table: object   # [B][max_blocks] int32
    seq_lens: object = None  # [B] int32

    def struct(self) -> MsaKvCache:
        return MsaKvCache(_p(self.k_pages), _p(self.v_pages), _p(self.summaries),
                          _p(self.block_table), _p(self.seq_lens),
                          int(self.k_pages.shape[0]), int(self.block_table.shape[-1]))


def _p(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream, like) -> Optional[int]:
    if stream is not None:
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return int(torch.cuda.current_stream(like.device).cuda_stream)


def _check(status: int, where: str) -> None:
    if status != MSA_OK:
        raise MsaError(status, where)


def msa_workspace_size(cfg: MsaConfig, op: int, batch: int, max_seq_len: int, chunk_len: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().msa_workspace_size(ctypes.byref(cfg), op, batch, max_seq_len, chunk_len,
                                             ctypes.byref(n)), "msa_workspace_size")
    return int(n.value)


def _workspace(cfg, op, batch, max_seq_len, chunk_len, workspace, like):
    need = msa_workspace_size(cfg, op, batch, max_seq_len, chunk_len)
    if workspace is None:
        import torch
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=like.device)
    return workspace, int(workspace.numel() * workspace.element_size())


def msa_build_summaries(cfg: MsaConfig, cache: KVCache, batch: int, max_seq_len: int, stream=None) -> None:
    c = cache.struct()
    _check(load_library().msa_build_summaries(ctypes.byref(cfg), ctypes.byref(c), batch, max_seq_len,
                                              _stream(stream, cache.k_pages)), "msa_build_summaries")


def msa_score(cfg: MsaConfig, q, cache: KVCache, batch: int, max_seq_len: int, scores_out,
              stream=None) -> None:
    c = cache.struct()
    _check(load_library().msa_score(ctypes.byref(cfg), _p(q), ctypes.byref(c), batch, max_seq_len,
                                    _p(scores_out), _stream(stream, q)), "msa_score")


def msa_select(cfg: MsaConfig, q, cache: KVCache, batch: int, max_seq_len: int, idx_out,
               scores_out=None, workspace=None, stream=None) -> None:
    ws, nbytes = _workspace(cfg, MSA_OP_SELECT, batch, max_seq_len, 0, workspace, q)
    c = cache.struct()
    _check(load_library().msa_select(ctypes.byref(cfg), _p(q), ctypes.byref(c), batch, max_seq_len,
                                     _p(scores_out), _p(idx_out), _p(ws), nbytes, _stream(stream, q)),
           "msa_select")


def msa_select_index(cfg: MsaConfig, q_index, index_keys, block_table, seq_lens, batch: int,
                     max_seq_len: int, idx_out, scores_out=None, workspace=None, stream=None) -> None:
    """q_index [batch][Hkv][128], index_keys [num_pages][64][128] (cfg's dtype), paged through
    block_table [batch][max_blocks]; only the table, lengths and page count reach the cache struct."""
    ws, nbytes = _workspace(cfg, MSA_OP_SELECT, batch, max_seq_len, 0, workspace, q_index)
    c = MsaKvCache(None, None, None, _p(block_table), _p(seq_lens), int(index_keys.shape[0]),
                   int(block_table.shape[-1]))
    _check(load_library().msa_select_index(ctypes.byref(cfg), _p(q_index), _p(index_keys),
                                           int(q_index.shape[-1]), ctypes.byref(c), batch, max_seq_len,
                                           _p(scores_out), _p(idx_out), _p(ws), nbytes,
                                           _stream(stream, q_index)), "msa_select_index")


def msa_attend(cfg: MsaConfig, q, cache: KVCache, batch: int, max_seq_len: int, idx, out,
               lse_out=None, workspace=None, stream=None) -> None:
    ws, nbytes = _workspace(cfg, MSA_OP_ATTEND, batch, max_seq_len, 0, workspace, q)
    c = cache.struct()
    _check(load_library().msa_attend(ctypes.byref(cfg), _p(q), ctypes.byref(c), batch, max_seq_len,
                                     _p(idx), _p(out), _p(lse_out), _p(ws), nbytes, _stream(stream, q)),
           "msa_attend")


def msa_decode_step(cfg: MsaConfig, q, cache: KVCache, batch: int, max_seq_len: int, out,
                    k_new=None, v_new=None, idx_out=None, scores_out=None, lse_out=None,
                    workspace=None, stream=None) -> None:
    ws, nbytes = _workspace(cfg, MSA_OP_DECODE, batch, max_seq_len, 0, workspace, q)
    c = cache.struct()
    _check(load_library().msa_decode_step(ctypes.byref(cfg), _p(q), ctypes.byref(c), batch, max_seq_len,
                                          _p(k_new), _p(v_new), _p(idx_out), _p(scores_out), _p(out),
                                          _p(lse_out), _p(ws), nbytes, _stream(stream, q)),
           "msa_decode_step")


def msa_decode_step_noalloc(cfg: MsaConfig, q, cache: KVCache, batch: int, max_seq_len: int, out, k_new=None,
                            v_new=None, idx_out=None, scores_out=None, lse_out=None, stream=None) -> None:
    """msa_decode_step with the library's own per-GPU scratch array as the workspace (no allocation)."""
    c = cache.struct()
    _check(load_library().msa_decode_step_noalloc(ctypes.byref(cfg), _p(q), ctypes.byref(c), batch, max_seq_len,
                                                  _p(k_new), _p(v_new), _p(idx_out), _p(scores_out), _p(out),
                                                  _p(lse_out), _stream(stream, q)),
           "msa_decode_step_noalloc")


NOALLOC_SCRATCH_BYTES = 32 << 20


def msa_prefill_chunk(cfg: MsaConfig, q, k_new, v_new, cache: KVCache, past_len: int, T: int, out,
                      idx_out=None, scores_out=None, lse_out=None, workspace=None, stream=None) -> None:
    ws, nbytes = _workspace(cfg, MSA_OP_PREFILL, 1, past_len + T, T, workspace, q)
    c = cache.struct()
    _check(load_library().msa_prefill_chunk(ctypes.byref(cfg), _p(q), _p(k_new), _p(v_new), ctypes.byref(c),
                                            past_len, T, _p(idx_out), _p(scores_out), _p(out), _p(lse_out),
                                            _p(ws), nbytes, _stream(stream, q)),
           "msa_prefill_chunk")


def msa_prefill_attend(cfg: MsaConfig, q, cache: KVCache, past_len: int, T: int, idx, out, lse_out=None,
                       stream=None) -> None:
    c = cache.struct()
    _check(load_library().msa_prefill_attend(ctypes.byref(cfg), _p(q), ctypes.byref(c), past_len, T, _p(idx),
                                             _p(out), _p(lse_out), _stream(stream, q)),
           "msa_prefill_attend")


PROBE_READ_SINK_FLOATS = 2048 * 256


def msa_probe_hbm_read(buf, sink, stream=None) -> None:
    """Streaming read of the whole device tensor buf (bytes a multiple of 16); sink: a float32
    device tensor of PROBE_READ_SINK_FLOATS elements."""
    nbytes = int(buf.numel()) * int(buf.element_size())
    if int(sink.numel()) < PROBE_READ_SINK_FLOATS:
        raise ValueError("sink needs %d floats" % PROBE_READ_SINK_FLOATS)
    _check(load_library().msa_probe_hbm_read(_p(buf), nbytes, _p(sink), _stream(stream, buf)), "msa_probe_hbm_read")


def msa_probe_mfma_bf16(sink, workgroups: int, iters: int, stream=None) -> None:
    """bf16 MFMA chains: workgroups * 4 * iters * 4 * 32768 FLOP; sink: >= 4 * workgroups floats."""
    if int(sink.numel()) < 4 * workgroups:
        raise ValueError("sink needs %d floats" % (4 * workgroups))
    _check(load_library().msa_probe_mfma_bf16(_p(sink), int(workgroups), int(iters), _stream(stream, sink)),
           "msa_probe_mfma_bf16")
