"""C-ABI boundary checks that need no GPU: the library loads, exports every function that
include/msa.h declares, sizes workspaces, and rejects invalid calls on the host before any
HIP call (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

lib_mod = pytest.importorskip("long_context_sparse_select_amd._lib")
L = lib_mod
if not os.path.exists(L.library_path()):
    pytest.skip("libmsa.so is not built", allow_module_level=True)

FAKE = 0x1000  # never dereferenced: every call below fails validation first


def declared_functions(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:msa_status|const char\*)\s+(msa_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    lib = L.load_library()
    names = declared_functions()
    assert set(names) == set(L.EXPORTED)
    probes = declared_functions(os.path.join(ROOT, "include", "msa_probe.h"))
    assert set(probes) == set(L.EXPORTED_PROBES)
    for n in names + probes:
        assert hasattr(lib, n), n


def test_probe_argument_validation():
    lib = L.load_library()
    sink = ctypes.c_void_p(16)   # never dereferenced: every call below is rejected on the host
    assert lib.msa_probe_hbm_read(None, 1 << 20, sink, None) == L.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_hbm_read(ctypes.c_void_p(256), 100, sink, None) == L.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_hbm_read(ctypes.c_void_p(8), 1 << 20, sink, None) == L.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_hbm_read(ctypes.c_void_p(256), 1 << 20, None, None) == L.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_mfma_bf16(None, 8, 10, None) == L.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_mfma_bf16(sink, 0, 10, None) == L.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_mfma_bf16(sink, 8, 0, None) == L.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_mfma_bf16(sink, 70000, 10, None) == L.MSA_ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert L.msa_status_string(s).startswith("MSA_")
    assert "unknown" in L.msa_status_string(99)


def cfg(**kw):
    base = dict(num_q_heads=32, num_kv_heads=8, top_k=64, dtype="bf16")
    base.update(kw)
    return L.make_config(**base)


def ws_size(c, op, B=1, max_len=1 << 20, T=0):
    n = ctypes.c_size_t(0)
    st = L.load_library().msa_workspace_size(ctypes.byref(c), op, B, max_len, T, ctypes.byref(n))
    return st, n.value


def test_workspace_sizes():
    c = cfg()
    st, sel = ws_size(c, L.MSA_OP_SELECT)
    assert st == 0
    # scores: 8 rows x 16384 blocks, fp32
    assert sel == 8 * 16384 * 4
    st, att = ws_size(c, L.MSA_OP_ATTEND)
    assert st == 0 and att > 0
    st, dec = ws_size(c, L.MSA_OP_DECODE)
    assert st == 0 and dec >= sel + att
    st, pre = ws_size(c, L.MSA_OP_PREFILL, 1, 262144 + 4096, 4096)
    assert st == 0 and pre > 0
    assert ws_size(c, L.MSA_OP_PREFILL, 2, 4096, 64)[0] == L.MSA_ERR_INVALID_ARG
    assert ws_size(c, 17)[0] == L.MSA_ERR_INVALID_ARG


def _prefill_base(Hq, Hkv, k, max_len, T):
    """the unsplit prefill workspace: scores, tile queries and lists (256-aligned arrays)"""
    a = lambda x: (x + 255) // 256 * 256
    rows = (T + 63) // 64 * Hkv
    return a(rows * ((max_len + 63) // 64) * 4) + a(rows * 128 * 4) + a(rows * (k + 1) * 4)


@pytest.mark.parametrize("Hq,Hkv,k,T", [(32, 8, 32, 4096), (32, 8, 32, 2048), (32, 8, 32, 1024), (32, 8, 32, 512),
                                        (32, 8, 32, 64), (64, 8, 32, 1024), (64, 8, 32, 2048), (8, 1, 64, 300),
                                        (32, 8, 1, 64), (32, 8, 2, 64), (32, 8, 3, 64), (4, 4, 4096, 64)])
def test_prefill_split_workspace(Hq, Hkv, k, T):
    """Short chunks split every tile's list over several workgroups so that about 256 workgroups
    run (1 when (tiles x groups x head splits) already reaches 256), at least two list slots per
    split and at most 256 splits; the workspace then also holds T * Hq * splits partials of
    128 + 2 floats."""
    hsplit = 2 if Hq // Hkv > 4 else 1
    units = (T + 63) // 64 * Hkv * hsplit
    want = 1 if units >= 256 else max(1, min(-(-256 // units), (k + 1) // 2, 256))
    max_len = 262144 + T
    st, pre = ws_size(cfg(num_q_heads=Hq, num_kv_heads=Hkv, top_k=k), L.MSA_OP_PREFILL, 1, max_len, T)
    assert st == 0
    a = lambda x: (x + 255) // 256 * 256
    extra = 0 if want == 1 else a(T * Hq * want * 128 * 4) + a(T * Hq * want * 2 * 4)
    assert pre == _prefill_base(Hq, Hkv, k, max_len, T) + extra


@pytest.mark.parametrize("B,Hq,Hkv", [(1, 8, 1), (1, 4, 2), (1, 32, 8), (2, 8, 1), (3, 16, 8), (8, 32, 8),
                                      (31, 32, 8), (32, 32, 8), (300, 8, 1)])
def test_attend_splits_fit_one_merge_workgroup(B, Hq, Hkv):
    """The attend workspace holds B * Hq * nsplit partials of 128 + 2 floats (two 256-aligned
    arrays); one merge workgroup combines at most 256 splits, so for every k the workspace must
    stay within 256 splits' worth (a 257th split would add B * Hq * 520 bytes, more than the
    alignment slack)."""
    for k in list(range(1, 1100)) + list(range(1100, 4097, 37)) + [4096]:
        c = cfg(num_q_heads=Hq, num_kv_heads=Hkv, top_k=k)
        st, att = ws_size(c, L.MSA_OP_ATTEND, B, 1 << 20)
        assert st == 0
        assert att <= B * Hq * 256 * (128 + 2) * 4 + 510, (B, Hq, Hkv, k)


@pytest.mark.parametrize("field,value,status", [
    ("num_q_heads", 0, L.MSA_ERR_INVALID_ARG),
    ("num_q_heads", 30, L.MSA_ERR_INVALID_ARG),        # Hq % Hkv != 0
    ("num_kv_heads", 2, L.MSA_ERR_UNSUPPORTED),       # group of 16 > 8
    ("top_k", 0, L.MSA_ERR_INVALID_ARG),
    ("top_k", 5000, L.MSA_ERR_UNSUPPORTED),
    ("head_dim", 64, L.MSA_ERR_UNSUPPORTED),
    ("block_size", 128, L.MSA_ERR_UNSUPPORTED),
    ("q_dtype", 7, L.MSA_ERR_INVALID_ARG),
    ("kv_dtype", 0, L.MSA_ERR_UNSUPPORTED),            # mixed q / kv types
    ("score_mode", 1, L.MSA_ERR_UNSUPPORTED),          # block max pool: msa_select_index only
    ("score_mode", 5, L.MSA_ERR_INVALID_ARG),
    ("keep_local", -1, L.MSA_ERR_INVALID_ARG),
    ("keep_sink", -1, L.MSA_ERR_INVALID_ARG),
    ("keep_local", 65, L.MSA_ERR_INVALID_ARG),         # forced blocks beyond top_k = 64
    ("keep_sink", 64, L.MSA_OK),
    ("keep_local", 64, L.MSA_OK),
    ("q_tile", 32, L.MSA_ERR_UNSUPPORTED),
    ("softmax_scale", float("nan"), L.MSA_ERR_INVALID_ARG),
    ("softmax_scale", -0.5, L.MSA_ERR_INVALID_ARG),
    ("softmax_scale", 0.0, L.MSA_ERR_INVALID_ARG),
])
def test_config_validation(field, value, status):
    c = cfg()
    setattr(c, field, value)
    assert ws_size(c, L.MSA_OP_DECODE)[0] == status


def test_forced_blocks_must_fit_in_k():
    assert ws_size(cfg(top_k=4, keep_sink=2, keep_local=2), L.MSA_OP_DECODE)[0] == L.MSA_OK
    assert ws_size(cfg(top_k=4, keep_sink=3, keep_local=2), L.MSA_OP_DECODE)[0] == L.MSA_ERR_INVALID_ARG


def fake_cache(max_blocks=16, num_pages=16, **kw):
    c = L.MsaKvCache(FAKE, FAKE, FAKE, FAKE, FAKE, num_pages, max_blocks)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def call_decode(c, cache, B=1, max_len=1024, q=FAKE, out=FAKE, k_new=None, v_new=None, ws=FAKE, nbytes=1 << 30):
    return L.load_library().msa_decode_step(ctypes.byref(c), q, ctypes.byref(cache), B, max_len, k_new, v_new,
                                            None, None, out, None, ws, nbytes, None)


def test_decode_argument_errors():
    c = cfg()
    ok_cache = fake_cache()
    assert call_decode(c, ok_cache, q=None) == L.MSA_ERR_INVALID_ARG
    assert call_decode(c, ok_cache, out=None) == L.MSA_ERR_INVALID_ARG
    assert call_decode(c, ok_cache, k_new=FAKE) == L.MSA_ERR_INVALID_ARG          # v_new missing
    assert call_decode(c, ok_cache, B=-1) == L.MSA_ERR_INVALID_ARG
    assert call_decode(c, ok_cache, max_len=16 * 64 + 1) == L.MSA_ERR_INVALID_ARG  # beyond the table
    assert call_decode(c, ok_cache, B=65536) == L.MSA_ERR_UNSUPPORTED               # beyond the grid limit
    assert ws_size(c, L.MSA_OP_DECODE, B=65536)[0] == L.MSA_ERR_UNSUPPORTED
    assert ws_size(c, L.MSA_OP_DECODE, B=65535, max_len=1024)[0] == L.MSA_OK
    assert call_decode(c, fake_cache(k_pages=None)) == L.MSA_ERR_INVALID_ARG
    assert call_decode(c, fake_cache(seq_lens=None)) == L.MSA_ERR_INVALID_ARG
    assert call_decode(c, fake_cache(max_blocks=0)) == L.MSA_ERR_INVALID_ARG
    assert call_decode(c, ok_cache, ws=None) == L.MSA_ERR_WORKSPACE
    assert call_decode(c, ok_cache, nbytes=16) == L.MSA_ERR_WORKSPACE
    bad = cfg(top_k=0)
    assert call_decode(bad, ok_cache) == L.MSA_ERR_INVALID_ARG


def test_select_attend_build_errors():
    lib = L.load_library()
    c = cfg()
    cache = fake_cache()
    assert lib.msa_select(ctypes.byref(c), FAKE, ctypes.byref(cache), 1, 1024, None, None, FAKE, 1 << 30, None) == L.MSA_ERR_INVALID_ARG
    assert lib.msa_select(ctypes.byref(c), FAKE, ctypes.byref(cache), 1, 1024, None, FAKE, FAKE, 8, None) == L.MSA_ERR_WORKSPACE
    assert lib.msa_attend(ctypes.byref(c), FAKE, ctypes.byref(cache), 1, 1024, None, FAKE, None, FAKE, 1 << 30, None) == L.MSA_ERR_INVALID_ARG
    nokv = fake_cache(v_pages=None)
    assert lib.msa_attend(ctypes.byref(c), FAKE, ctypes.byref(nokv), 1, 1024, FAKE, FAKE, None, FAKE, 1 << 30, None) == L.MSA_ERR_INVALID_ARG
    assert lib.msa_build_summaries(ctypes.byref(c), ctypes.byref(fake_cache(summaries=None)), 1, 1024, None) == L.MSA_ERR_INVALID_ARG
    assert lib.msa_build_summaries(ctypes.byref(c), ctypes.byref(cache), 1, 5000, None) == L.MSA_ERR_INVALID_ARG


def test_prefill_errors():
    lib = L.load_library()
    cache = fake_cache(max_blocks=80, num_pages=80)

    def call(c, past=1024, T=256, q=FAKE, nbytes=1 << 30):
        return lib.msa_prefill_chunk(ctypes.byref(c), q, FAKE, FAKE, ctypes.byref(cache), past, T, None, None,
                                     FAKE, None, FAKE, nbytes, None)
    assert call(cfg(), past=1000) == L.MSA_ERR_UNSUPPORTED       # past_len % 64 != 0
    assert call(cfg(), T=0) == L.MSA_ERR_INVALID_ARG
    assert call(cfg(), past=80 * 64, T=1) == L.MSA_ERR_INVALID_ARG  # beyond the table
    assert call(cfg(), q=None) == L.MSA_ERR_INVALID_ARG
    assert call(cfg(dtype="f32")) == L.MSA_ERR_UNSUPPORTED       # prefill is bf16 only
    assert call(cfg(), nbytes=100) == L.MSA_ERR_WORKSPACE


def test_decode_noalloc_errors():
    """msa_decode_step_noalloc validates like msa_decode_step and rejects a decode whose workspace
    would exceed its scratch array, before any HIP call (none of these calls touches a device)."""
    lib = L.load_library()

    def call(c=None, B=1, max_len=1024, cache=None, q=FAKE, out=FAKE, k_new=None, v_new=None):
        c = cfg() if c is None else c
        cache = fake_cache() if cache is None else cache
        return lib.msa_decode_step_noalloc(ctypes.byref(c), q, ctypes.byref(cache), B, max_len, k_new, v_new, None,
                                           None, out, None, None)
    assert call(q=None) == L.MSA_ERR_INVALID_ARG
    assert call(out=None) == L.MSA_ERR_INVALID_ARG
    assert call(k_new=FAKE) == L.MSA_ERR_INVALID_ARG          # k_new without v_new
    assert call(max_len=5000) == L.MSA_ERR_INVALID_ARG        # beyond the table
    assert call(c=cfg(head_dim=64)) == L.MSA_ERR_UNSUPPORTED
    assert call(B=0) == L.MSA_OK
    # the limit: the same layout as msa_workspace_size reports for a decode step
    big = fake_cache(max_blocks=1 << 16, num_pages=1 << 16)
    for B, max_len in [(1, 1 << 20), (32, 1 << 20), (1, 1 << 22), (64, 1 << 20), (8, 1 << 22)]:
        need = ws_size(cfg(), L.MSA_OP_DECODE, B, max_len)[1]
        st = call(B=B, max_len=max_len, cache=big, q=None)       # q = None: stops before any launch
        if need > L.NOALLOC_SCRATCH_BYTES:
            assert call(B=B, max_len=max_len, cache=big) == L.MSA_ERR_WORKSPACE, (B, max_len)
        assert st == L.MSA_ERR_INVALID_ARG
    assert ws_size(cfg(), L.MSA_OP_DECODE, 32, 1 << 20)[1] <= L.NOALLOC_SCRATCH_BYTES
    assert ws_size(cfg(), L.MSA_OP_DECODE, 64, 1 << 20)[1] > L.NOALLOC_SCRATCH_BYTES


def test_prefill_attend_errors():
    """msa_prefill_attend reads only the table, page count and K/V pools of the cache (no
    summaries, no lengths, no workspace)."""
    lib = L.load_library()
    bare = fake_cache(max_blocks=80, num_pages=80, summaries=None, seq_lens=None)

    def call(c=None, past=1024, T=256, q=FAKE, idx=FAKE, out=FAKE, cache=bare):
        c = cfg() if c is None else c
        return lib.msa_prefill_attend(ctypes.byref(c), q, ctypes.byref(cache), past, T, idx, out, None, None)
    assert call(past=1000) == L.MSA_ERR_UNSUPPORTED       # past_len % 64 != 0
    assert call(T=0) == L.MSA_ERR_INVALID_ARG
    assert call(past=-64) == L.MSA_ERR_INVALID_ARG
    assert call(past=80 * 64, T=1) == L.MSA_ERR_INVALID_ARG
    assert call(q=None) == L.MSA_ERR_INVALID_ARG
    assert call(idx=None) == L.MSA_ERR_INVALID_ARG
    assert call(out=None) == L.MSA_ERR_INVALID_ARG
    assert call(cache=fake_cache(max_blocks=80, num_pages=80, k_pages=None)) == L.MSA_ERR_INVALID_ARG
    assert call(cache=fake_cache(max_blocks=80, num_pages=80, block_table=None)) == L.MSA_ERR_INVALID_ARG
    assert call(c=cfg(dtype="f32")) == L.MSA_ERR_UNSUPPORTED
    assert call(c=cfg(head_dim=64)) == L.MSA_ERR_UNSUPPORTED


def test_select_index_errors():
    """The index branch reads only the table, lengths and page count of the cache; index_dim
    other than 64 or 128 is unsupported; score_mode is not read."""
    lib = L.load_library()
    bare = fake_cache(k_pages=None, v_pages=None, summaries=None)

    def call(c=None, qi=FAKE, ik=FAKE, di=128, cache=bare, B=1, max_len=1024, idx=FAKE, nbytes=1 << 30, ws=FAKE):
        c = cfg() if c is None else c
        return lib.msa_select_index(ctypes.byref(c), qi, ik, di, ctypes.byref(cache), B, max_len, None, idx, ws,
                                    nbytes, None)
    assert call(qi=None) == L.MSA_ERR_INVALID_ARG
    assert call(ik=None) == L.MSA_ERR_INVALID_ARG
    assert call(idx=None) == L.MSA_ERR_INVALID_ARG
    assert call(di=0) == L.MSA_ERR_INVALID_ARG
    assert call(di=96) == L.MSA_ERR_UNSUPPORTED
    assert call(di=64, B=0) == L.MSA_OK          # 64 and 128 are both accepted
    assert call(cache=fake_cache(seq_lens=None)) == L.MSA_ERR_INVALID_ARG
    assert call(cache=fake_cache(block_table=None)) == L.MSA_ERR_INVALID_ARG
    assert call(max_len=16 * 64 + 1) == L.MSA_ERR_INVALID_ARG
    assert call(B=-1) == L.MSA_ERR_INVALID_ARG
    assert call(nbytes=8) == L.MSA_ERR_WORKSPACE
    assert call(ws=None) == L.MSA_ERR_WORKSPACE
    assert call(c=cfg(top_k=0)) == L.MSA_ERR_INVALID_ARG
    # a valid call with no sequences enqueues nothing and succeeds, in either score mode
    assert call(B=0) == L.MSA_OK
    assert call(B=0, c=cfg(score_mode=1)) == L.MSA_OK
    # the config-driven select still refuses the max-token mode
    assert lib.msa_select(ctypes.byref(cfg(score_mode=1)), FAKE, ctypes.byref(fake_cache()), 1, 1024, None, FAKE,
                          FAKE, 1 << 30, None) == L.MSA_ERR_UNSUPPORTED


def test_summary_dtype_validation():
    assert ws_size(cfg(summary_dtype="bf16"), L.MSA_OP_DECODE)[0] == L.MSA_OK
    c = cfg()
    c.summary_dtype = 7
    assert ws_size(c, L.MSA_OP_DECODE)[0] == L.MSA_ERR_INVALID_ARG


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MSA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m is not None
    assert int(m.group(1)) << int(m.group(2)) == L.NOALLOC_SCRATCH_BYTES
