"""The streaming-read probe (a measurement aid) reads every byte it is given:
the XOR of its per-workgroup words equals the XOR of the buffer's words."""

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_06_amd import router as rt

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,sink_words", [(16, 1), (1051664, 8192), (1051664, 7), (64 << 20, 8192)])
def test_probe_reads_every_word(nbytes, sink_words):
    dev = torch.device("cuda:0")
    rt.load_library()
    gen = torch.Generator(device=dev).manual_seed(nbytes)
    buf = torch.randint(-(1 << 31), 1 << 31, (nbytes // 4,), dtype=torch.int64, device=dev, generator=gen)
    buf = buf.to(torch.int32)
    sink = torch.zeros(sink_words, dtype=torch.int32, device=dev)
    rt.probe_read(buf, sink)
    torch.cuda.synchronize()
    grid = min((nbytes // 16 + 255) // 256, sink_words, 8192)
    got = np.bitwise_xor.reduce(sink[:grid].cpu().numpy())
    want = np.bitwise_xor.reduce(buf.cpu().numpy())
    assert got == want


def test_mfma_probe_runs_the_same_work_everywhere():
    dev = torch.device("cuda:0")
    rt.load_library()
    sink = torch.full((rt.MFMA_PROBE_SINK,), float("nan"), dtype=torch.float32, device=dev)
    rt.probe_mfma(64, sink)
    torch.cuda.synchronize()
    v = sink.cpu().numpy().reshape(1024, 256)
    assert np.all(np.isfinite(v))
    assert np.all(v == v[0][None, :])  # every workgroup computed the same sums
