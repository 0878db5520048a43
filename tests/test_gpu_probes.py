"""GPU checks of the measurement probes (include/msa_probe.h): the streaming-read probe reads
every 16-byte element exactly once (a single non-zero element shows up in exactly the thread
that owns it), and the MFMA probe's work scales exactly with its round count."""
import numpy as np
import pytest
import torch

import long_context_sparse_select_amd as msa
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("n16,i", [(1, 0), (4096, 4095), (300000, 123457), (2048 * 2048 + 5, 2048 * 2048 + 3)])
def test_read_probe_sees_each_element_once(n16, i):
    words = np.zeros((n16, 4), np.uint32)
    words[i] = [0x12345678, 0x0000ffff, 0x00ff0000, 0x1]
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((msa.PROBE_READ_SINK_FLOATS,), -1.0, dtype=torch.float32, device="cuda")
    msa.msa_probe_hbm_read(buf, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy()
    # element e is read by thread e % 256 of workgroup (e // 2048) % 2048 (eight 256-element rows
    # per workgroup per round, 2048 workgroups per round)
    owner = ((i // 2048) % 2048) * 256 + i % 256
    want = float((0x12345678 ^ 0x0000ffff ^ 0x00ff0000 ^ 0x1) & 0xffff)
    assert got[owner] == want
    others = np.delete(got, owner)
    assert np.all(others == 0.0)


def test_mfma_probe_scales_with_rounds():
    sink10 = torch.zeros(4 * 16, dtype=torch.float32, device="cuda")
    sink20 = torch.zeros_like(sink10)
    msa.msa_probe_mfma_bf16(sink10, 16, 10)
    msa.msa_probe_mfma_bf16(sink20, 16, 20)
    torch.cuda.synchronize()
    a, b = sink10.cpu().numpy(), sink20.cpu().numpy()
    assert np.all(np.isfinite(a)) and np.any(a != 0.0)
    np.testing.assert_array_equal(b, 2.0 * a)   # dyadic operands: every partial sum is exact
