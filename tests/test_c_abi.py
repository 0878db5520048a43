"""The C ABI from plain C: tests/c/abi_decode_check.c includes only msa.h and the HIP runtime's C
API, links libmsa.so (and, as the checker, liboracle.so), runs one fp32 decode step and compares
it with the oracle. The CPU test compiles it (msa.h is valid C; the library's symbols resolve);
the GPU test runs it."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "long_context_sparse_select_amd")
ORC = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out_dir):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    if not os.path.exists(os.path.join(PKG, "libmsa.so")) or not os.path.exists(os.path.join(ORC, "liboracle.so")):
        pytest.skip("libmsa.so / liboracle.so not built")
    exe = os.path.join(str(out_dir), "abi_decode_check")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
           os.path.join(HERE, "c", "abi_decode_check.c"), "-o", exe,
           "-L" + PKG, "-lmsa", "-L" + ORC, "-loracle", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath," + PKG, "-Wl,-rpath," + ORC, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_builds_against_the_abi(tmp_path):
    build(tmp_path)


@pytest.mark.gpu
def test_c_program_decode_step_matches_oracle(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = build(tmp_path)
    print("running the C ABI decode check", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout.strip(), flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout, r.stdout
