"""gq_linear_noalloc (no workspace argument, no allocation: the library's
static per-GPU scratch) against gq_linear with a caller workspace, through
the C ABI.  Both run the same kernels with the same launch plans, so the
outputs must be identical bit for bit.  Two calls in a row on the shared
scratch, the second with a smaller input, for each path that uses scratch
(small-batch split K, prefill GEMM) and for the dot-product path (none)."""
import numpy as np
import pytest
import torch

import synth as S

pytestmark = pytest.mark.gpu

gq = pytest.importorskip("quantized_gemm_groupwise_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def _packed(N, K, bits, block_n, seed):
    W = torch.from_numpy(S.decode_weight(0, N=N, K=K, seed_base=seed)).cuda()
    return gq.quantize_pack(W, bits, block_n)


def _pair(p, M, seed):
    """(y from gq_linear with a fresh workspace, y from gq_linear_noalloc)."""
    x = torch.from_numpy(S.activations(M, p.K, seed).view(np.int16)).cuda().view(torch.bfloat16)
    need = gq.gq_linear_workspace_bytes(p.layout, M)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    y_ref = torch.full((M, p.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    y_na = torch.full((M, p.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = gq.gq_linear(p.layout, M, gq.GQ_BF16, x.data_ptr(), p.codes.data_ptr(), p.scales.data_ptr(),
                      p.zeros.data_ptr(), y_ref.data_ptr(), ws.data_ptr(), ws.numel())
    assert st == gq.GQ_OK, gq.gq_status_string(st)
    st = gq.gq_linear_noalloc(p.layout, M, gq.GQ_BF16, x.data_ptr(), p.codes.data_ptr(),
                              p.scales.data_ptr(), p.zeros.data_ptr(), y_na.data_ptr())
    assert st == gq.GQ_OK, gq.gq_status_string(st)
    torch.cuda.synchronize()
    return need, y_ref.view(torch.int16).cpu().numpy(), y_na.view(torch.int16).cpu().numpy()


# (N, K, bits, block_n, M) of the first call, then of the second, smaller call
CASES = [
    # small-batch path with K split across workgroups (fp32 partials in scratch)
    ((4096, 14336, [4], None, 24), (256, 28672, [2], None, 9)),
    # prefill GEMM (fp16 activations, row exponents, split parts in scratch)
    ((2048, 4096, [4, 2] * 8, 128, 512), (768, 1024, [2, 4, 2, 4, 2, 4], 128, 72)),
    # dot-product path: no scratch at all
    ((4096, 4096, [4], None, 3), (1024, 4096, [2], None, 1)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_linear_twice(first, second):
    needs = []
    for i, (N, K, bits, block_n, M) in enumerate((first, second)):
        print("noalloc case", N, K, bits[:2], block_n, M, flush=True)
        p = _packed(N, K, bits, block_n, 9100 + 10 * i + M)
        need, y_ref, y_na = _pair(p, M, 9200 + M)
        assert need <= gq.GQ_NOALLOC_SCRATCH_BYTES
        needs.append(need)
        assert np.array_equal(y_ref, y_na), f"call {i}: {(y_ref != y_na).sum()} outputs differ"
        # every output written (the buffers start as NaN)
        f = (y_na.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        assert np.isfinite(f).all()
    assert needs[1] <= needs[0]


def test_noalloc_too_large_refused_on_gpu():
    lay = gq.make_layout(28672, 8192, 8192, [2])
    st = gq.gq_linear_noalloc(lay, 2048, gq.GQ_BF16, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000)
    assert st == gq.GQ_ERR_TOO_LARGE
