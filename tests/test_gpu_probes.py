"""The measurement probes bench.py reports attainable peaks with: the
streaming read sees every byte (the XOR of its sink values equals the XOR of
all 32-bit words of the buffer, bit for bit), and the MFMA loop gives every
workgroup the same finite value."""
import functools

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (4096, 3), (1 << 20, 64), ((1 << 20) + 48, 7), (3 << 24, 2048)])
def test_probe_read_sees_every_byte(gpu_lib, nbytes, wgs):
    import torch
    rng = np.random.default_rng(nbytes + wgs)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    dev = torch.from_numpy(host.view(np.int32)).cuda()
    sink = gpu_lib.probe_hbm_read(dev, workgroups=wgs)
    got = functools.reduce(np.bitwise_xor, sink.cpu().numpy().view(np.uint32), np.uint32(0))
    assert got == np.bitwise_xor.reduce(host)


def test_probe_mfma_uniform(gpu_lib):
    sink = gpu_lib.probe_mfma_bf16(64, workgroups=300).cpu().numpy()
    assert np.all(np.isfinite(sink)) and np.all(sink == sink[0]) and sink[0] != 0.0


def test_probe_rejects(gpu_lib):
    import torch
    with pytest.raises(Exception):
        gpu_lib.probe_hbm_read(torch.zeros(10, dtype=torch.uint8, device="cuda"))   # 10 bytes: not a multiple of 16
