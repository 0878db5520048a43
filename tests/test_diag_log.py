"""Launch logging (MSA_LOG): host-side only, so the entry point that needs no GPU,
msa_workspace_size, checks it here; the GPU test in test_gpu_diag.py covers kernel launches.
The variable is read once per process, so every case runs in a child interpreter."""
import os
import subprocess
import sys

import pytest

pytest.importorskip("long_context_sparse_select_amd._lib")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SNIPPET = r"""
import sys
sys.path.insert(0, %r)
import long_context_sparse_select_amd as msa
cfg = msa.make_config(32, 8, 64, dtype="bf16")
print(msa.msa_workspace_size(cfg, msa.MSA_OP_DECODE, 1, 1 << 20))
print(msa.msa_workspace_size(cfg, msa.MSA_OP_PREFILL, 1, 266240, 4096))
""" % ROOT


def run(env_value):
    env = dict(os.environ)
    env.pop("MSA_LOG", None)
    if env_value is not None:
        env["MSA_LOG"] = env_value
    r = subprocess.run([sys.executable, "-c", SNIPPET], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr
    sizes = [int(x) for x in r.stdout.split()]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[msa]")]
    return sizes, lines


@pytest.mark.parametrize("value", [None, "", "0"])
def test_log_off(value):
    _, lines = run(value)
    assert lines == []


def test_log_on_names_the_call_and_its_result():
    sizes, lines = run("1")
    assert lines == ["[msa] msa_workspace_size: op %d, batch 1, max_seq_len %d -> %d B" % (2, 1 << 20, sizes[0]),
                     "[msa] msa_workspace_size: prefill, max_seq_len 266240, chunk 4096 -> %d B" % sizes[1]]
