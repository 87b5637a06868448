"""The benchmark's streaming-read probe (libgq_probe.so, the one-launch read
ceiling bench.py reports next to the decode fractions) runs on the GPU,
reads without writing the buffer, and leaves its sink alone for ordinary
data."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(os.path.join(ROOT, "quantized_gemm_groupwise_amd", "libgq_probe.so"))
    fn = lib.gqprobe_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


@pytest.mark.parametrize("nbytes", [16, 4096, 16400, 72550400])
def test_stream_probe_reads(probe, nbytes):
    print("stream probe", nbytes, flush=True)
    buf = torch.arange(nbytes // 4, dtype=torch.int32, device="cuda")
    before = buf.clone()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = probe(buf.data_ptr(), nbytes, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(buf, before)
    assert int(sink[1:].abs().sum().item()) == 0
