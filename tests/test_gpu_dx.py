"""GPU parity of the data gradient dX = dY . W_hat (gq_linear_dx) against the
CPU oracle (oracle.linear_dx, fp64) on the same seeded inputs.

Bar, as for the forward matmul: normwise relative error <= 2e-3 against the
fp64 oracle and the elementwise bound
|dx - dx_ref| <= 2^-8 |dx_ref| + 2^-10 sum_n |dy_n| |w_hat_nk|
(bf16 output rounding, one fp16 rounding per weight, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

gq = pytest.importorskip("quantized_gemm_groupwise_amd")
from tests.gpu_util import bf16_dev, to_dev, upload_packed, y_bits  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def _say(*a):
    print(*a, flush=True)


def grad(M, N, seed):
    """Synthetic output gradient: bf16 bits, Gaussian with a per-row scale
    spread over two decades (rows of a real dY differ in magnitude; a wider
    spread would leave a sampled normwise error to a handful of rows)."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((M, N)) * 10.0 ** rng.uniform(-2, 0, size=(M, 1))
    return S.bf16_bits(g.astype(np.float32))


def dx_gate(dx_bits, dx_ref, dy_bits, w_abs, fp16_out=False):
    """w_abs: |W_hat| [N][k] for the compared columns."""
    if fp16_out:
        dg = dx_bits.view(np.float16).astype(np.float64)
        da = np.abs(dy_bits.view(np.float16).astype(np.float64))
    else:
        dg = O.bf16_bits_to_f64(dx_bits)
        da = np.abs(O.bf16_bits_to_f64(dy_bits))
    normwise = np.linalg.norm(dg - dx_ref) / np.linalg.norm(dx_ref)
    assert normwise <= 2e-3, normwise
    bound = 2.0 ** -8 * np.abs(dx_ref) + 2.0 ** -10 * (da @ w_abs)
    bad = np.abs(dg - dx_ref) > bound
    assert not bad.any(), f"{bad.sum()} elements outside the bound"
    return normwise


@pytest.mark.parametrize("M,N,K,block_n,bits", [
    (1, 512, 512, 512, [4]),                  # one row
    (40, 200, 1024, 200, [2]),                # N not a multiple of the 128-row step
    (256, 384, 768, 128, [2, 4, 2]),          # one full tile row, Channel-mix steps
    (300, 136, 576, 136, [2]),                # ragged M, K % 256 != 0: idle waves
    (520, 1024, 512, 128, [4, 2, 2, 4, 4, 2, 4, 2]),   # three m tiles
    (64, 8192, 256, 128, [4, 2] * 32),        # one tile: n split across workgroups
    (33, 4096, 640, 4096, [4]),               # split n, ragged M and K
])
def test_linear_dx_shapes(M, N, K, block_n, bits):
    W = S.decode_weight(4, N=N, K=K)
    ref = O.quantize_pack(W, O.Layout(K, N, block_n, bits))
    p = upload_packed(ref)
    dy = grad(M, N, 60 + M)
    _say("dx", M, N, K, len(bits), "blocks")
    dx = gq.linear_dx(bf16_dev(dy), p)
    torch.cuda.synchronize()
    assert dx.shape == (M, K) and dx.dtype == torch.bfloat16
    dx_gate(y_bits(dx), O.linear_dx(dy, ref), dy, np.abs(O.dequant(ref).astype(np.float64)))


def test_linear_dx_fp16():
    M, N, K = 70, 512, 256
    W = S.decode_weight(2, N=N, K=K)
    ref = O.quantize_pack(W, O.Layout(K, N, 128, [4, 2, 4, 4]))
    p = upload_packed(ref)
    dyf = np.random.default_rng(8).standard_normal((M, N)).astype(np.float16)
    dx = gq.linear_dx(to_dev(dyf), p)
    torch.cuda.synchronize()
    assert dx.dtype == torch.float16
    dref = dyf.astype(np.float64) @ O.dequant(ref).astype(np.float64)
    dx_gate(dx.cpu().numpy().view(np.uint16), dref, dyf.view(np.uint16),
            np.abs(O.dequant(ref).astype(np.float64)), fp16_out=True)


def test_linear_dx_exact_integer_case():
    """dY in {-1, 0, 1} with 31 nonzeros per row and weights on a 2^-6 grid:
    every dX is an integer times 2^-6 below 256 x 2^-6, exact in bf16, so
    the result must be bit-exact (across two m tiles and a split n)."""
    rng = np.random.default_rng(31)
    M, N, K = 300, 2048, 384
    base = rng.integers(-7, 9, size=(N, K)).astype(np.float64)
    base[:, 0::128] = -7
    base[:, 1::128] = 8
    W = (base * 2.0 ** -6).astype(np.float32)
    ref = O.quantize_pack(W, O.Layout(K, N, N, [4]))
    p = upload_packed(ref)
    di = np.zeros((M, N), dtype=np.int64)
    for m in range(M):
        pos = rng.choice(N, 31, replace=False)
        di[m, pos] = rng.choice([-1, 1], size=31)
    dy = S.bf16_bits(di.astype(np.float32))
    dx = gq.linear_dx(bf16_dev(dy), p)
    torch.cuda.synchronize()
    exact = (di @ base.astype(np.int64)) * 2.0 ** -6
    assert np.abs(exact).max() / 2 ** -6 < 256
    assert np.array_equal(O.bf16_bits_to_f64(y_bits(dx)), exact)


def test_linear_dx_is_the_adjoint_of_linear():
    """<dY, x . W_hat^T> = <dY . W_hat, x> with both products from the GPU,
    to the rounding of the two bf16 outputs."""
    M, N, K = 260, 640, 1024
    W = S.decode_weight(6, N=N, K=K)
    p = gq.quantize_pack(to_dev(W), [4, 2, 2, 4, 2], 128)
    x = bf16_dev(S.activations(M, K, 5))
    dy = bf16_dev(grad(M, N, 6))
    y = gq.linear(x, p).double()
    dx = gq.linear_dx(dy, p).double()
    lhs = (dy.double() * y).sum().item()
    rhs = (dx * x.double()).sum().item()
    # each side carries one bf16 rounding per output element (<= 2^-9
    # relative) over the same fp16-rounded weights
    scale = (dy.double().abs() * y.abs()).sum().item() + (dx.abs() * x.double().abs()).sum().item()
    assert abs(lhs - rhs) <= 2 ** -8 * scale


def test_linear_dx_degenerate_and_errors():
    K = 256
    p = gq.quantize_pack(to_dev(S.decode_weight(3, N=128, K=K)), 4)
    dx = gq.linear_dx(torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda"), p)
    assert dx.shape == (0, K)
    # N == 0: an empty sum
    p0 = gq.quantize_pack(torch.zeros((0, K), dtype=torch.float32, device="cuda"), 4)
    out = torch.full((5, K), 7.0, dtype=torch.bfloat16, device="cuda")
    gq.linear_dx(torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda"), p0, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    # N % 8 != 0 is refused on the host
    p12 = gq.quantize_pack(to_dev(S.decode_weight(3, N=12, K=K)), 4)
    with pytest.raises(gq.GqError) as e:
        gq.linear_dx(torch.zeros((4, 12), dtype=torch.bfloat16, device="cuda"), p12)
    assert e.value.status == gq.GQ_ERR_SHAPE


def test_linear_dx_repeat_and_shared_workspace():
    """Bitwise deterministic; one workspace serves a split and an unsplit
    call in turn."""
    N, K = 4096, 512
    p = gq.quantize_pack(to_dev(S.decode_weight(0, N=N, K=K)), [4, 2] * 16, 128)
    dys = [bf16_dev(grad(M, N, M)) for M in (64, 700)]
    need = max(gq.gq_linear_dx_workspace_bytes(p.layout, d.shape[0]) for d in dys)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    first = [y_bits(gq.linear_dx(d, p, ws=ws)) for d in dys]
    second = [y_bits(gq.linear_dx(d, p, ws=ws)) for d in reversed(dys)][::-1]
    for a, b in zip(first, second):
        assert np.array_equal(a, b)


def _sampled_dx_check(W, bits, block_n, dy, dxb, ms, wins, rng, ncols=16):
    """dX at rows ms and sampled columns of the 128-column windows wins; the
    oracle quantizes each window alone (128 is a multiple of both group
    sizes, so a window holds whole groups of every row)."""
    N = W.shape[0]
    got, want, bw = [], [], []
    for w0 in wins:
        c0 = 128 * w0
        ref = O.quantize_pack(np.ascontiguousarray(W[:, c0:c0 + 128]), O.Layout(128, N, block_n, bits))
        cols = sorted(set(rng.choice(128, ncols, replace=False).tolist()) | {0, 127})
        want.append(O.linear_dx(dy[ms], ref, cols))
        got.append(dxb[np.ix_(ms, [c0 + c for c in cols])])
        bw.append(np.abs(O.dequant(ref).astype(np.float64))[:, cols])
    want = np.concatenate(want, 1)
    rounding = np.linalg.norm(O.bf16_bits_to_f64(O.f64_to_bf16_bits(want)) - want) / np.linalg.norm(want)
    _say("normwise", dx_gate(np.concatenate(got, 1), want, dy[ms], np.concatenate(bw, 1)),
         "bf16 rounding of the exact result alone", rounding)


@pytest.mark.parametrize("N,bits", [(8192, [4]), (8192, [4, 2, 2, 2] * 16)])
def test_linear_dx_tail_split(N, bits):
    """M = 2048, K = 8448: 264 tiles of 256 x 256, so the last 8 (columns
    8192..8447) are cut along n into 4 parts and summed by the tail
    reduction."""
    M, K = 2048, 8448
    block_n = N if len(bits) == 1 else 128
    W = S.decode_weight(8, N=N, K=K)
    _say("dx tail split", M, N, K, len(bits), "blocks")
    p = gq.quantize_pack(torch.from_numpy(W).cuda(), bits, block_n)
    dy = grad(M, N, 71)
    dxb = y_bits(gq.linear_dx(bf16_dev(dy), p))
    torch.cuda.synchronize()
    rng = np.random.default_rng(72)
    ms = sorted(set(rng.choice(M, 24, replace=False).tolist()) | {0, M - 1})
    wins = [0, 17, 63, 64, 65]                 # 64 and 65: the split tail tiles
    _sampled_dx_check(W, bits, block_n, dy, dxb, ms, wins, rng)


@pytest.mark.parametrize("j", [0, 1])
def test_linear_dx_channel_mix_full_size(j):
    """The 70B-class MLP linears (Channel-mix INT4/INT2 blocks of 128
    channels) at M = 2048, as the benchmark launches them: dX[m][k] at sampled
    (m, k).  Column k needs every row's group that holds k; the 128-column
    window around k holds exactly those groups (128 is a multiple of both
    group sizes), so the oracle quantizes that window alone."""
    N, K = S.MLP70B_SHAPES[j]
    W, bits = S.channel_mix_weight(j)
    _say("dx channel-mix", j, N, K)
    p = gq.quantize_pack(torch.from_numpy(W).cuda(), bits, 128)
    M = 2048
    dy = grad(M, N, 90 + j)
    dx = gq.linear_dx(bf16_dev(dy), p)
    torch.cuda.synchronize()
    dxb = y_bits(dx)
    rng = np.random.default_rng(40 + j)
    # two rows of every 256-row band of m and one 128-column window in every
    # 256-column band of k: every 256 x 256 tile of dX (the tail-split tiles
    # of the last round included) holds sampled outputs
    ms = sorted({int(t + rng.integers(256)) for t in range(0, M, 256) for _ in range(2)} | {0, M - 1})
    wins = sorted({2 * t + int(rng.integers(2)) for t in range(K // 256)} | {0, K // 128 - 1})
    _sampled_dx_check(W, bits, 128, dy, dxb, ms, wins, rng, ncols=4)
