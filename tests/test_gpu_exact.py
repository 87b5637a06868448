"""Bit-exact INT2 (and mixed INT4/INT2) cases on every matmul path, a
regression case for an MFMA operand hazard in the small-batch path, and
activation rows far from unit magnitude on the paths that rescale them.

Exact cases: weights on a power-of-two grid whose groups span exactly the
code range, activations in {-1, 0, 1}.  Every product and partial sum is then
an integer times a power of two that fp32 holds exactly, and each output is
below 256 units of the grid, so it is a bf16 value: the GPU result must equal
the exact value bit for bit, on the dot-product (M <= 4), small-batch MFMA
(4 < M <= 32), tiled GEMM (M > 32, both tile sizes) and dX kernels.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

gq = pytest.importorskip("quantized_gemm_groupwise_amd")
from tests.gpu_util import bf16_dev, upload_packed, y_bits  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def _say(*a):
    print(*a, flush=True)


U = 2.0 ** -6           # grid of the exact weights


def exact_weights(rng, N, K, block_n, bits):
    """Integers b with every group spanning exactly the code range (INT4
    [-7, 8], INT2 [-1, 2]), so S = U and z = 7 / 1: W = b * U exactly, and
    the oracle's dequantized weights equal W."""
    base = np.zeros((N, K), dtype=np.int64)
    for blk, b in enumerate(bits):
        r0 = blk * block_n
        lo, hi = (-7, 8) if b == 4 else (-1, 2)
        g = O.GROUP_SIZE[b]
        part = rng.integers(lo, hi + 1, size=(block_n, K))
        part[:, 0::g] = lo
        part[:, 1::g] = hi
        base[r0:r0 + block_n] = part
    return base


def exact_acts(rng, M, K, nnz):
    xi = np.zeros((M, K), dtype=np.int64)
    for m in range(M):
        pos = rng.choice(K, nnz, replace=False)
        xi[m, pos] = rng.choice([-1, 1], size=nnz)
    return xi


CASES = [
    # (M, N, K, block_n, bits): dot-product, small batch, GEMM, 256 x 256 GEMM
    (1, 192, 512, 192, [2]),
    (3, 256, 1024, 128, [2, 4]),
    (4, 200, 1536, 200, [2]),                # matrix-core decode path, ragged rows, 1.5 slices
    (8, 192, 512, 192, [2]),
    (24, 384, 2048, 128, [2, 4, 2]),
    (32, 128, 28672, 128, [2]),              # long k range: small-batch K split
    (96, 256, 512, 128, [4, 2]),
    (300, 16384, 256, 16384, [2]),           # 256 x 256 tiles
]


@pytest.mark.parametrize("M,N,K,block_n,bits", CASES)
def test_linear_exact_integer_int2(M, N, K, block_n, bits):
    rng = np.random.default_rng(500 + M)
    base = exact_weights(rng, N, K, block_n, bits)
    W = (base * U).astype(np.float32)
    ref = O.quantize_pack(W, O.Layout(K, N, block_n, bits))
    assert np.array_equal(O.dequant(ref).astype(np.float64), base * U)
    xi = exact_acts(rng, M, K, 100)          # |y| / U <= 100 * 8 ... capped below
    if 4 in bits:
        xi = exact_acts(rng, M, K, 31)       # INT4 blocks: |y| / U <= 31 * 8 < 256
    exact = (xi @ base.T) * U
    assert np.abs(exact).max() / U < 256
    p = upload_packed(ref)
    _say("exact", M, N, K, bits[:3])
    y = gq.linear(bf16_dev(S.bf16_bits(xi.astype(np.float32))), p)
    torch.cuda.synchronize()
    assert np.array_equal(O.bf16_bits_to_f64(y_bits(y)), exact)


def test_linear_dx_exact_integer_int2():
    rng = np.random.default_rng(531)
    M, N, K = 300, 2048, 384
    bits = [2, 4] * 8
    base = exact_weights(rng, N, K, 128, bits)
    W = (base * U).astype(np.float32)
    ref = O.quantize_pack(W, O.Layout(K, N, 128, bits))
    di = exact_acts(rng, M, N, 31)
    exact = (di @ base) * U
    assert np.abs(exact).max() / U < 256
    dx = gq.linear_dx(bf16_dev(S.bf16_bits(di.astype(np.float32))), upload_packed(ref))
    torch.cuda.synchronize()
    assert np.array_equal(O.bf16_bits_to_f64(y_bits(dx)), exact)


@pytest.mark.parametrize("M", [1, 4, 8, 16, 24, 32, 64])
def test_int2_one_code_distinct_scales(M):
    """Every code 1, every zero point 0, a different power-of-two scale per
    group (2^-(j mod 16)), activations non-zero in one group per row (group
    m mod 32, the last group included): y[m][n] = S_{n,j} * sum of that
    group's activations, exact in bf16.  The small-batch kernel once lost
    the last step of its INT2 tiles here, when an unpack instruction the
    compiler could not see overwrote a register an MFMA still read."""
    N, K = 256, 2048
    G = K // 64
    lay = O.Layout(K, N, N, [2])
    codes = O.pack(np.ones((N, K), dtype=np.uint8), 2)
    j = np.arange(G)
    sc = np.tile((2.0 ** -(j % 16)).astype(np.float16), (N, 1))
    ref = O.Packed(lay, codes.astype("<u4").view(np.uint8).reshape(-1).copy(),
                   sc.view(np.uint16).reshape(-1).copy(), np.zeros(N * G, dtype=np.uint8), 0)
    rng = np.random.default_rng(600 + M)
    xi = np.zeros((M, K), dtype=np.int64)
    for m in range(M):
        g = (m * 7 + 31) % G if m else G - 1
        xi[m, 64 * g:64 * g + 64] = rng.choice([-1, 0, 1], size=64)
    exact = np.zeros((M, N))
    for m in range(M):
        g = (m * 7 + 31) % G if m else G - 1
        exact[m, :] = xi[m, 64 * g:64 * g + 64].sum() * 2.0 ** -(g % 16)
    assert np.array_equal(O.linear(S.bf16_bits(xi.astype(np.float32)), ref), exact)
    y = gq.linear(bf16_dev(S.bf16_bits(xi.astype(np.float32))), upload_packed(ref))
    torch.cuda.synchronize()
    assert np.array_equal(O.bf16_bits_to_f64(y_bits(y)), exact)


def _rows(kind, M, K, seed):
    """bf16 activation rows: Gaussian times 2^60, times 2^-60, or times a
    ramp over 2^-20 .. 2^20 along the row (a row spanning 2^40)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    if kind == "huge":
        x *= 2.0 ** 60
    elif kind == "tiny":
        x *= 2.0 ** -60
    else:
        x *= 2.0 ** np.linspace(-20, 20, K)[None, :]
        x = x[:, rng.permutation(K)]
    return S.bf16_bits(x.astype(np.float32))


def _gate(got_bits, ref, a_bits, wabs):
    got = O.bf16_bits_to_f64(got_bits)
    normwise = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert normwise <= 2e-3, normwise
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -10 * (np.abs(O.bf16_bits_to_f64(a_bits)) @ wabs)
    assert np.all(np.abs(got - ref) <= bound), int((np.abs(got - ref) > bound).sum())
    return normwise


@pytest.mark.parametrize("kind", ["huge", "tiny", "span"])
@pytest.mark.parametrize("M", [1, 4, 8, 64, 300])
def test_linear_activation_range(kind, M):
    """The GEMM rescales each bf16 row by a power of two into fp16; the other
    paths use bf16 as given.  Rows at 2^60, at 2^-60 and spanning 2^40."""
    N, K = (16384, 256) if M == 300 else (256, 1024)
    bits = [4, 2] * (N // 256)
    W = S.decode_weight(3, N=N, K=K)
    ref = O.quantize_pack(W, O.Layout(K, N, 128, bits))
    x = _rows(kind, M, K, 700 + M)
    y = gq.linear(bf16_dev(x), upload_packed(ref))
    torch.cuda.synchronize()
    cols = np.arange(N) if N <= 256 else np.random.default_rng(1).choice(N, 256, replace=False)
    wd = O.dequant(ref, cols).astype(np.float64)
    y_ref = O.bf16_bits_to_f64(x) @ wd.T
    _say(kind, M, _gate(y_bits(y)[:, cols], y_ref, x, np.abs(wd).T))


@pytest.mark.parametrize("kind", ["huge", "tiny", "span"])
def test_linear_dx_gradient_range(kind):
    """dX rescales each bf16 row of dY by a power of two into fp16."""
    M, N, K = 300, 512, 384
    bits = [2, 4, 4, 2]
    W = S.decode_weight(4, N=N, K=K)
    ref = O.quantize_pack(W, O.Layout(K, N, 128, bits))
    dy = _rows(kind, M, N, 800)
    dx = gq.linear_dx(bf16_dev(dy), upload_packed(ref))
    torch.cuda.synchronize()
    wd = O.dequant(ref).astype(np.float64)
    _say(kind, _gate(y_bits(dx), O.bf16_bits_to_f64(dy) @ wd, dy, np.abs(wd)))
