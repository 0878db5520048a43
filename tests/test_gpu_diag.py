"""Launch logging on the GPU: a child process with MSA_LOG=1 runs one decode step (bf16, 1 x 38,400
tokens, 32 q / 8 kv heads, k = 16, with a new token); its stderr must name the entry point with
the chosen layout and every kernel the step launches, and its outputs must equal those of the
same step run here without logging (the log changes nothing on the device)."""
import os
import re
import subprocess
import sys

import numpy as np
import pytest
import torch

from gpu_util import require_gpu, run_decode, to_device
from synth import make_decode_case

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def step_outputs():
    c = make_decode_case(B=1, Hq=32, Hkv=8, lens=[38400], top_k=16, dtype="bf16", seed=71)
    d = to_device(c)
    g = torch.Generator(device="cuda")
    g.manual_seed(72)
    kn = torch.randn((1, 8, 128), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((1, 8, 128), generator=g, device="cuda").to(torch.bfloat16)
    r = run_decode(d, k_new=kn, v_new=vn)
    return {k: v.float().cpu().numpy() if v.dtype != torch.int32 else v.cpu().numpy() for k, v in r.items()}


CHILD = r"""
import sys
sys.path[:0] = [%r, %r]
import numpy as np
from test_gpu_diag import step_outputs
r = step_outputs()
np.savez(sys.argv[1], **r)
""" % (ROOT, HERE)


def test_log_of_a_decode_step(tmp_path):
    require_gpu()
    out_file = str(tmp_path / "child.npz")
    env = dict(os.environ, MSA_LOG="1")
    print("child: decode step with MSA_LOG=1", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, out_file], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[msa]")]
    text = "\n".join(lines)
    assert re.search(r"msa_build_summaries: batch 1, max_seq_len 38400, 8 kv heads, f32 summaries", text), text
    assert re.search(r"msa_decode_step: batch 1, max_seq_len 38400, 32 q / 8 kv heads, top_k 16, bf16; row stride 600, "
                     r"\d+ split\(s\) of \d+ block\(s\), top-k inside the attend launch; workspace \d+ of \d+ B, "
                     r"appending a new token", text), text
    for kernel in (r"k_build_summaries<bf16 keys, f32 summaries>",
                   r"k_score_decode<bf16 q, Hkv=8, f32 summaries, with the new token's append, run maxima> "
                   r"grid 46 x 1 x 1, 256 threads",
                   r"k_decode_select_attend<G=4, blocks in flight \d> grid \d+ x 8 x 1, 256 threads",
                   r"k_merge<bf16, splits/8 = \d+> grid 32 x 1 x 1, 256 threads"):
        assert re.search(r"\[msa\]   launch " + kernel, text), (kernel, text)
    # the step's own launches, in order
    step = lines[[i for i, l in enumerate(lines) if "msa_decode_step:" in l][0] + 1:]
    assert [re.search(r"launch (\w+)<", l).group(1) for l in step] == ["k_score_decode", "k_decode_select_attend",
                                                                         "k_merge"]
    child = np.load(out_file)
    here = step_outputs()
    for k in ("o", "lse", "idx", "scores"):
        np.testing.assert_array_equal(child[k], here[k], err_msg=k)


def check_scenarios():
    """Run in a child with MSA_DEVICE_CHECKS=1: (status, outputs) per scenario."""
    import long_context_sparse_select_amd as msa
    res = {}

    def status_of(fn):
        try:
            fn()
            torch.cuda.synchronize()
            return 0
        except msa.MsaError as e:
            return e.status
    # clean data: the step runs and its outputs match the unchecked run (compared by the parent)
    r = step_outputs()
    res["clean"] = r
    # a page id out of range in a visible block of sequence 1
    c = make_decode_case(B=2, Hq=8, Hkv=2, lens=[700, 2000], top_k=8, dtype="bf16", seed=73)
    c.block_table = c.block_table.copy()
    c.block_table[1, 5] = c.num_pages + 3
    d = to_device(c, build=False)
    res["bad_page"] = status_of(lambda: run_decode(d))
    # a length beyond max_seq_len
    c2 = make_decode_case(B=2, Hq=8, Hkv=2, lens=[700, 2000], top_k=8, dtype="bf16", seed=74)
    d2 = to_device(c2)
    d2.lens[0] = 2000 + 64
    res["bad_len"] = status_of(lambda: run_decode(d2))
    # an attend list that repeats a block
    c3 = make_decode_case(B=1, Hq=8, Hkv=2, lens=[3000], top_k=8, dtype="bf16", seed=75)
    d3 = to_device(c3)
    idx = torch.tensor([[[3, 9, 12, -1, 40, 9, 2, 7], [0, 1, 2, 3, 4, 5, 6, 7]]], dtype=torch.int32, device="cuda")
    out = torch.empty_like(d3.q)
    res["repeat"] = status_of(lambda: msa.msa_attend(d3.cfg, d3.q, d3.cache, 1, c3.max_seq_len, idx, out))
    idx_ok = idx.clone()
    idx_ok[0, 0, 5] = 11
    res["no_repeat"] = status_of(lambda: msa.msa_attend(d3.cfg, d3.q, d3.cache, 1, c3.max_seq_len, idx_ok, out))
    # under graph capture the check stands aside (it would have to synchronise)
    c4 = make_decode_case(B=1, Hq=8, Hkv=2, lens=[3000], top_k=8, dtype="bf16", seed=76)
    d4 = to_device(c4)
    out4 = torch.empty_like(d4.q)
    ws = torch.empty(msa.msa_workspace_size(d4.cfg, msa.MSA_OP_DECODE, 1, c4.max_seq_len), dtype=torch.uint8,
                     device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        msa.msa_decode_step(d4.cfg, d4.q, d4.cache, 1, c4.max_seq_len, out4, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()

    def capture():
        with torch.cuda.graph(g):
            msa.msa_decode_step(d4.cfg, d4.q, d4.cache, 1, c4.max_seq_len, out4, workspace=ws)
        g.replay()
    res["captured"] = status_of(capture)
    return res


CHECK_CHILD = r"""
import sys, pickle
sys.path[:0] = [%r, %r]
import numpy as np
from test_gpu_diag import check_scenarios
r = check_scenarios()
np.savez(sys.argv[1], **r.pop("clean"))
open(sys.argv[2], "w").write(repr(r))
""" % (ROOT, HERE)


def test_device_checks(tmp_path):
    require_gpu()
    import long_context_sparse_select_amd as msa
    out_file, st_file = str(tmp_path / "clean.npz"), str(tmp_path / "status.txt")
    env = dict(os.environ, MSA_DEVICE_CHECKS="1")
    env.pop("MSA_LOG", None)
    print("child: device-check scenarios with MSA_DEVICE_CHECKS=1", flush=True)
    r = subprocess.run([sys.executable, "-c", CHECK_CHILD, out_file, st_file], capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    status = eval(open(st_file).read())
    assert status == {"bad_page": msa.MSA_ERR_INVALID_ARG, "bad_len": msa.MSA_ERR_INVALID_ARG,
                      "repeat": msa.MSA_ERR_INVALID_ARG, "no_repeat": 0, "captured": 0}, status
    lines = [l for l in r.stderr.splitlines() if l.startswith("[msa]")]
    c = make_decode_case(B=2, Hq=8, Hkv=2, lens=[700, 2000], top_k=8, dtype="bf16", seed=73)
    assert len(lines) == 3, lines
    assert lines[0] == ("[msa] MSA_DEVICE_CHECKS: msa_decode_step: block_table[1][5] = %d is not a page id in "
                        "[0, num_pages)" % (c.num_pages + 3)), lines
    assert lines[1] == ("[msa] MSA_DEVICE_CHECKS: msa_decode_step: seq_lens[0] = 2064 is outside "
                        "[0, min(max_seq_len, max_blocks * 64)]"), lines
    # either occurrence of the repeated block may be the one reported
    assert re.fullmatch(r"\[msa\] MSA_DEVICE_CHECKS: msa_attend: idx\[0\]\[0\]\[(1|5)\] = 9 repeats a block already "
                        r"listed in its row", lines[2]), lines
    child = np.load(out_file)
    here = step_outputs()
    for k in ("o", "lse", "idx", "scores"):
        np.testing.assert_array_equal(child[k], here[k], err_msg=k)
