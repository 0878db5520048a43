"""Two-stage GQA block-sparse attention on MI355X (gfx950): Python binding of libmsa.

Argument marshalling only: every step runs in the HIP kernels of libmsa.so, reached through
its C ABI (include/msa.h) with ctypes. torch supplies device memory and the current stream.
There is no CPU fallback; calling any entry point without the built library raises.

Entry points (same names as the C ABI):
  msa_workspace_size, msa_build_summaries, msa_score, msa_select, msa_select_index, msa_attend,
  msa_decode_step, msa_decode_step_noalloc, msa_prefill_chunk, msa_prefill_attend, msa_status_string
Measurement probes of the GPU itself (include/msa_probe.h): msa_probe_hbm_read, msa_probe_mfma_bf16
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    MSA_BF16, MSA_F32, MSA_OP_ATTEND, MSA_OP_DECODE, MSA_OP_PREFILL, MSA_OP_SELECT, KVCache,
    MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP,
    MsaError, library_path, load_library, make_config, msa_attend, msa_build_summaries,
    msa_decode_step, msa_decode_step_noalloc, msa_prefill_attend, msa_prefill_chunk, msa_score, msa_select, msa_select_index, msa_status_string,
    msa_workspace_size, msa_probe_hbm_read, msa_probe_mfma_bf16, PROBE_READ_SINK_FLOATS, NOALLOC_SCRATCH_BYTES,
)

__all__ = [
    "MSA_BF16", "MSA_F32", "MSA_OP_ATTEND", "MSA_OP_DECODE", "MSA_OP_PREFILL", "MSA_OP_SELECT",
    "MSA_OK", "MSA_ERR_INVALID_ARG", "MSA_ERR_UNSUPPORTED", "MSA_ERR_WORKSPACE", "MSA_ERR_HIP",
    "KVCache", "MsaError", "library_path", "load_library", "make_config", "msa_attend",
    "msa_build_summaries", "msa_decode_step", "msa_decode_step_noalloc", "msa_prefill_attend", "msa_prefill_chunk", "msa_score", "msa_select",
    "msa_select_index", "msa_status_string", "msa_workspace_size",
    "msa_probe_hbm_read", "msa_probe_mfma_bf16", "PROBE_READ_SINK_FLOATS", "NOALLOC_SCRATCH_BYTES",
]
