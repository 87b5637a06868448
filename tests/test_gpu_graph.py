"""The library's calls captured in a HIP graph (as the benchmark times them)
give, on every replay, the bytes of the same call run eagerly.  Replays are
separated by eager work and synchronisations; the calls that split their
reduction (fp32 parts in the workspace) are among them."""
import numpy as np
import pytest
import torch

import synth as S

pytestmark = pytest.mark.gpu

gq = pytest.importorskip("quantized_gemm_groupwise_amd")
from tests.gpu_util import bf16_dev, to_dev  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def _bytes(t):
    return t.view(torch.uint8).cpu().numpy().copy()


def _graph_matches_eager(fn, out):
    """fn() writes into out; capture it, replay 3 times, compare each replay
    with the eager result."""
    fn()
    torch.cuda.synchronize()
    want = _bytes(out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(0)
        junk = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bytes(out), want), f"replay {r} differs from the eager result"
        del junk


@pytest.mark.parametrize("M", [1, 12, 300])
def test_linear_in_graph(M):
    N, K = 1024, 4096
    p = gq.quantize_pack(to_dev(S.decode_weight(0, N=N, K=K)), [4, 2] * 4, 128)
    x = bf16_dev(S.activations(M, K, 3))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = gq.workspace(gq.gq_linear_workspace_bytes(p.layout, M), "cuda")
    _graph_matches_eager(lambda: gq.linear(x, p, out=y, ws=ws), y)


@pytest.mark.parametrize("M,N,K", [(64, 8192, 512), (2048, 8192, 8448)])
def test_linear_dx_in_graph(M, N, K):
    """An n-split (64 rows, one tile) and a tail split (264 tiles)."""
    p = gq.quantize_pack(to_dev(S.decode_weight(1, N=N, K=K)), [4, 2] * (N // 256), 128)
    rng = np.random.default_rng(4)
    dy = bf16_dev(S.bf16_bits((rng.standard_normal((M, N)) * 0.1).astype(np.float32)))
    dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    ws = gq.workspace(gq.gq_linear_dx_workspace_bytes(p.layout, M), "cuda")
    _graph_matches_eager(lambda: gq.linear_dx(dy, p, out=dx, ws=ws), dx)


def test_fake_quant_in_graph():
    N, K = 512, 1024
    W = to_dev(S.decode_weight(2, N=N, K=K))
    lay = gq.make_layout(K, N, 128, [4, 2, 2, 4])
    out = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    _graph_matches_eager(lambda: gq.gq_fake_quant(lay, W.data_ptr(), gq.GQ_BF16, out.data_ptr()), out)


def test_kv_attention_in_graph():
    """Packed splits, window parts and the combine, captured and replayed."""
    B, Hq, Hkv, tp, tw = 2, 32, 8, 700, 40
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    k = torch.randn((B * tp, Hkv * 128), generator=gen, device="cuda")
    v = torch.randn((B * tp, Hkv * 128), generator=gen, device="cuda")
    kp, vp = gq.quantize_pack(k, 4), gq.quantize_pack(v, 4)
    kw = torch.randn((B, tw, Hkv, 128), generator=gen, device="cuda").to(torch.bfloat16)
    vw = torch.randn((B, tw, Hkv, 128), generator=gen, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, Hq, 128), generator=gen, device="cuda").to(torch.bfloat16)
    o = torch.empty_like(q)
    cache = gq.kv_cache(B, Hq, Hkv, kp, vp, kw, vw)
    ws = gq.workspace(gq.gq_kv_attention_workspace_bytes(cache), "cuda")
    _graph_matches_eager(lambda: gq.kv_attention(q, cache, out=o, ws=ws), o)
