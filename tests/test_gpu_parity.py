"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bar: packed codes, scales, zeros and flags byte-identical; dequantized
weights bit-identical; linear outputs within the normwise relative error
2e-3 against the fp64 oracle and within an elementwise bound
|y - y_ref| <= 2^-8 |y_ref| + 2^-10 sum_k |x_k| |w_hat_k|
(bf16 output rounding plus fp32 accumulation / one fp16 rounding per weight).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

gq = pytest.importorskip("quantized_gemm_groupwise_amd")
from tests.gpu_util import bf16_dev, gpu_quantize, to_dev, upload_packed, y_bits  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def _say(*a):
    print(*a, flush=True)


def assert_packed_equal(W, block_n, bits, check_flags=True):
    L = O.Layout(W.shape[1], W.shape[0], block_n, list(bits))
    ref = O.quantize_pack(W, L)
    codes, scales, zeros, flags, _ = gpu_quantize(W, block_n, list(bits))
    assert np.array_equal(codes, ref.codes), "codes differ"
    assert np.array_equal(scales, ref.scales), "scales differ"
    assert np.array_equal(zeros, ref.zeros), "zeros differ"
    if check_flags:
        assert flags == ref.flags
    return ref


def linear_gate(y_gpu_bits, y_ref, x_bits, op, fp16_out=False, rows=None):
    if fp16_out:
        yg = y_gpu_bits.view(np.float16).astype(np.float64)
    else:
        yg = O.bf16_bits_to_f64(y_gpu_bits)
    denom = np.linalg.norm(y_ref)
    normwise = np.linalg.norm(yg - y_ref) / denom
    assert normwise <= 2e-3, normwise
    xa = np.abs(O.bf16_bits_to_f64(x_bits)) if not fp16_out else np.abs(x_bits.view(np.float16).astype(np.float64))
    wa = np.abs(O.dequant(op, rows).astype(np.float64))
    bound = 2.0 ** -8 * np.abs(y_ref) + 2.0 ** -10 * (xa @ wa.T)
    bad = np.abs(yg - y_ref) > bound
    assert not bad.any(), f"{bad.sum()} elements outside the bound"
    return normwise


# ------------------------------------------------------------- quantize

def test_quantize_small_layer():
    d = S.small_layer()
    _say("quantize 512x512 INT4")
    assert_packed_equal(d["W"], 512, [4])


@pytest.mark.parametrize("N,K,block_n,bits", [
    (1, 128, 1, [4]), (3, 640, 3, [4]), (129, 576, 129, [2]), (64, 64, 64, [2]),
    (512, 1024, 128, [4, 2, 2, 4]), (384, 256, 128, [2, 4, 2]), (256, 8192, 256, [2]),
])
def test_quantize_shapes(N, K, block_n, bits):
    W = S.decode_weight(1, N=N, K=K)
    _say("quantize", N, K, block_n, bits)
    assert_packed_equal(W, block_n, bits)


def test_quantize_edge_groups():
    """Degenerate groups, exact ties, fp16-subnormal scales, scale overflow,
    non-finite inputs (codes of a non-finite group are unspecified)."""
    g = 128
    rows = []
    rows.append(np.full(g, 0.37, np.float32))                     # hi == lo
    rows.append(np.full(g, -2.6, np.float32))
    r = np.zeros(g, np.float32); r[1] = 15 * (1 + 2 ** -11); rows.append(r)     # scale tie
    r = np.zeros(g, np.float32); r[1] = 15 * 3 * 2 ** -26; rows.append(r)       # subnormal scale
    r = np.zeros(g, np.float32); r[1] = 15 * 2.0 ** -25; rows.append(r)         # scale -> 0 -> 1
    r = (np.arange(g, dtype=np.float32) - 40.5) * np.float32(2 ** -7); rows.append(r)  # ties
    r = np.linspace(3.0, 4.0, g, dtype=np.float32); rows.append(r)              # z clamps to 0
    r = np.linspace(-4.0, -3.0, g, dtype=np.float32); rows.append(r)            # z clamps to 15
    r = np.zeros(g, np.float32); r[3] = 1e-39; r[4] = -3e-40; rows.append(r)    # fp32 denormals
    W = np.stack(rows)
    _say("quantize edge groups")
    assert_packed_equal(W, W.shape[0], [4])
    W2 = np.stack([W[0], W[2]])
    W2[1, 7] = 15 * 65520.0                                       # fp16 overflow -> flag
    ref = assert_packed_equal(W2, 2, [4])
    assert ref.flags == O.FLAG_SCALE_OVERFLOW
    W3 = np.stack([W[5], W[6]])
    W3[1, 9] = np.nan
    L = O.Layout(g, 2, 2, [4])
    ref = O.quantize_pack(W3, L)
    codes, scales, zeros, flags, _ = gpu_quantize(W3, 2, [4])
    assert flags == O.FLAG_NONFINITE == ref.flags
    assert np.array_equal(codes[:64], ref.codes[:64]) and scales[0] == ref.scales[0] and zeros[0] == ref.zeros[0]


def test_quantize_flags_accumulate_and_inf():
    g = 64
    W = np.zeros((2, g), np.float32)
    W[0, 0] = np.inf
    codes, scales, zeros, flags, p = gpu_quantize(W, 2, [2])
    assert flags == O.FLAG_NONFINITE


# ------------------------------------------------------------- dequant

@pytest.mark.parametrize("block_n,bits", [(256, [4]), (256, [2]), (128, [2, 4])])
def test_dequant_bit_exact(block_n, bits):
    W = S.decode_weight(2, N=256, K=512)
    L = O.Layout(512, 256, block_n, bits)
    ref = O.quantize_pack(W, L)
    p = upload_packed(ref)
    for dt, name in [(torch.float32, "fp32"), (torch.float16, "fp16"), (torch.bfloat16, "bf16")]:
        out = gq.dequant(p, dt)
        torch.cuda.synchronize()
        exp = O.dequant_as(ref, name)
        got = out.cpu()
        if name == "bf16":
            got = got.view(torch.int16).numpy().view(np.uint16)
        else:
            got = got.numpy()
        assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(exp).view(np.uint8)), name


# ------------------------------------------------------- fake quantization

def _fq_bytes(t: torch.Tensor, name: str) -> np.ndarray:
    got = t.cpu()
    got = got.view(torch.int16).numpy().view(np.uint16) if name == "bf16" else got.numpy()
    return np.ascontiguousarray(got).view(np.uint8)


@pytest.mark.parametrize("N,K,block_n,bits", [
    (1, 64, 1, [2]), (3, 640, 3, [4]), (129, 576, 129, [2]), (256, 1024, 256, [4]),
    (512, 1024, 128, [4, 2, 2, 4]), (384, 768, 128, [2, 4, 2]),
])
def test_fake_quant_bit_exact(N, K, block_n, bits):
    """gq_fake_quant equals the oracle's quantize-then-dequantize, bit for bit,
    for fp32, fp16 and bf16 outputs, and the GPU's own quantize_pack + dequant."""
    W = S.decode_weight(4, N=N, K=K)
    L = O.Layout(K, N, block_n, bits)
    w = to_dev(W)
    p = gq.quantize_pack(w, bits, block_n)
    _say("fake quant", N, K, block_n, bits)
    for dt, name in [(torch.float32, "fp32"), (torch.float16, "fp16"), (torch.bfloat16, "bf16")]:
        flags = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = gq.fake_quant(w, bits, block_n, dt, flags=flags)
        two_pass = gq.dequant(p, dt)
        torch.cuda.synchronize()
        exp = np.ascontiguousarray(O.fake_quant(W, L, name)).view(np.uint8)
        assert np.array_equal(_fq_bytes(out, name), exp), name
        assert np.array_equal(_fq_bytes(two_pass, name), exp), name
        assert int(flags.item()) == 0


def test_fake_quant_flags_and_edge_groups():
    """The flags of quantize_pack, and exact output for degenerate, clamped-zero
    and tie groups next to a non-finite one (whose output is unspecified)."""
    g = 128
    rows = [np.full(g, 0.37, np.float32), np.linspace(3.0, 4.0, g, dtype=np.float32),
            np.linspace(-4.0, -3.0, g, dtype=np.float32),
            (np.arange(g, dtype=np.float32) - 40.5) * np.float32(2 ** -7), np.zeros(g, np.float32)]
    W = np.stack(rows)
    W[4, 5] = np.nan
    L = O.Layout(g, W.shape[0], W.shape[0], [4])
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = gq.fake_quant(to_dev(W), 4, W.shape[0], torch.float32, flags=flags)
    torch.cuda.synchronize()
    exp = O.fake_quant(W, L)
    assert np.array_equal(out.cpu().numpy()[:4], exp[:4])
    # rows 1 and 2 do not straddle zero: their zero points clamp
    assert int(flags.item()) == O.FLAG_NONFINITE | O.FLAG_ZERO_CLAMPED == O.quantize_pack(W, L).flags


# ------------------------------------------------------------- linear

@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("N,K,block_n,bits", [
    (512, 512, 512, [4]), (300, 1024, 300, [2]), (1000, 2048, 1000, [4]),
    (512, 1024, 128, [4, 2, 2, 4]), (129, 192, 129, [2]),
    (640, 8192, 640, [4]),          # rows longer than one load group, 2 staging sub-units at M = 1
    (256, 6144, 128, [4, 2]),       # the same for a Channel-mix layout, 3-slice INT4 rows
])
def test_linear_gemv(M, N, K, block_n, bits):
    W = S.decode_weight(0, N=N, K=K)
    L = O.Layout(K, N, block_n, bits)
    ref = O.quantize_pack(W, L)
    p = upload_packed(ref)
    x = S.activations(M, K, 77 + M)
    _say("gemv", M, N, K, bits)
    y = gq.linear(bf16_dev(x), p)
    torch.cuda.synchronize()
    linear_gate(y_bits(y), O.linear(x, ref), x, ref)


@pytest.mark.parametrize("M", [5, 17, 32, 33, 64, 65, 130, 300])
@pytest.mark.parametrize("N,K,block_n,bits", [
    (512, 512, 512, [4]), (200, 1024, 200, [2]), (384, 768, 128, [2, 4, 2]),
    (136, 576, 136, [2]),          # K % 128 == 64: half k-step at the end
    (256, 4096, 128, [4, 2]),      # long K: split-K partials for small M
])
def test_linear_gemm(M, N, K, block_n, bits):
    W = S.decode_weight(3, N=N, K=K)
    L = O.Layout(K, N, block_n, bits)
    ref = O.quantize_pack(W, L)
    p = upload_packed(ref)
    x = S.activations(M, K, 500 + M)
    _say("gemm", M, N, K, bits)
    y = gq.linear(bf16_dev(x), p)
    torch.cuda.synchronize()
    linear_gate(y_bits(y), O.linear(x, ref), x, ref)


@pytest.mark.parametrize("M,N,K,block_n,bits", [
    (6, 16384, 256, 128, [4, 2] * 64),     # one k-way per workgroup, Channel-mix blocks
    (24, 14368, 320, 14368, [2]),          # two row blocks, ragged last tile, half k-step
    (12, 8192, 1152, 8192, [4]),           # two k-ways, last phase partly past the range
    (20, 7168, 1088, 7168, [2]),           # two k-ways, two row blocks, half k-step
    (9, 2048, 2944, 2048, [4]),            # four k-ways, ragged phases
    (7, 512, 8192, 512, [4]),              # narrow and long: K split across workgroups
    (30, 640, 1024, 128, [2, 4, 2, 2, 4]), # split K, Channel-mix, two row blocks
])
def test_linear_small_batch_shapes(M, N, K, block_n, bits):
    """4 < M <= 32 over the small-batch kernel's launch shapes (k-ways per
    workgroup, row blocks, split K) with ragged tails."""
    W = S.decode_weight(5, N=N, K=K)
    L = O.Layout(K, N, block_n, bits)
    ref = O.quantize_pack(W, L)
    p = upload_packed(ref)
    x = S.activations(M, K, 900 + M)
    _say("small batch", M, N, K, len(bits), "blocks")
    y = gq.linear(bf16_dev(x), p)
    torch.cuda.synchronize()
    linear_gate(y_bits(y), O.linear(x, ref), x, ref)


@pytest.mark.parametrize("M,N,K,block_n,bits", [
    (260, 16448, 192, 16448, [2]),                     # ragged M and N, half k-step
    (512, 16384, 256, 128, [4, 2, 2, 2] * 32),         # Channel-mix blocks
    (256, 32768, 128, 32768, [4]),                     # one 256-row tile
])
def test_linear_gemm_large_tiles(M, N, K, block_n, bits):
    """M >= 256 with >= 128 tiles: the 256 x 256 workgroup tile path."""
    W = S.decode_weight(1, N=N, K=K)
    L = O.Layout(K, N, block_n, bits)
    ref = O.quantize_pack(W, L)
    p = upload_packed(ref)
    x = S.activations(M, K, 900 + M)
    _say("gemm large tiles", M, N, K, len(bits), "blocks")
    y = gq.linear(bf16_dev(x), p)
    torch.cuda.synchronize()
    linear_gate(y_bits(y), O.linear(x, ref), x, ref)


def test_linear_exact_integer_case_large_tiles():
    """The exact case of test_linear_exact_integer_case on the 256 x 256 path."""
    rng = np.random.default_rng(77)
    M, N, K = 300, 32768, 256
    base = rng.integers(-7, 9, size=(N, K)).astype(np.float64)
    base[:, 0::128] = -7
    base[:, 1::128] = 8
    W = (base * 2.0 ** -6).astype(np.float32)
    ref = O.quantize_pack(W, O.Layout(K, N, N, [4]))
    p = upload_packed(ref)
    xi = np.zeros((M, K), dtype=np.float64)
    for m in range(M):
        pos = rng.choice(K, 31, replace=False)
        xi[m, pos] = rng.choice([-1.0, 1.0], size=31)
    x = S.bf16_bits(xi.astype(np.float32))
    y = gq.linear(bf16_dev(x), p)
    torch.cuda.synchronize()
    exact = (xi @ base.T) * 2.0 ** -6          # small integers: exact in fp64
    assert np.abs(exact).max() / 2 ** -6 < 256
    assert np.array_equal(O.bf16_bits_to_f64(y_bits(y)), exact)


@pytest.mark.parametrize("M,bits", [(2, 4), (20, 4), (70, 4), (3, 2), (4, 2)])
def test_linear_fp16_activations(M, bits):
    """fp16 activations; INT2 at M = 3-4 is the matrix-core decode path
    (its f16 4x4x4 products)."""
    N, K = 256, 512
    W = S.decode_weight(3, N=N, K=K)
    ref = O.quantize_pack(W, O.Layout(K, N, N, [bits]))
    p = upload_packed(ref)
    xf = np.random.default_rng(M).standard_normal((M, K)).astype(np.float16)
    # the oracle takes bf16 bit patterns; use fp16 values exact in fp64 instead
    y = gq.linear(to_dev(xf), p)
    torch.cuda.synchronize()
    yref = xf.astype(np.float64) @ O.dequant(ref).astype(np.float64).T
    yg = y.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(yg - yref) / np.linalg.norm(yref) <= 2e-3


@pytest.mark.parametrize("M", [1, 3, 8, 96])
def test_linear_exact_integer_case(M):
    """x in {-1,0,1}, weights on a power-of-two grid: y is exact in fp64 and
    exactly representable in bf16, so the GPU result must be bit-exact."""
    rng = np.random.default_rng(12 + M)
    N, K = 192, 512
    base = rng.integers(-7, 9, size=(N, K)).astype(np.float64)
    base[:, 0::128] = -7
    base[:, 1::128] = 8
    W = (base * 2.0 ** -6).astype(np.float32)
    ref = O.quantize_pack(W, O.Layout(K, N, N, [4]))
    p = upload_packed(ref)
    # 31 nonzero activations per row: |y| / 2^-6 <= 31 * 8 < 256, so every
    # exact result has at most 8 significant bits and is a bf16 value
    xi = np.zeros((M, K), dtype=np.int64)
    for m in range(M):
        pos = rng.choice(K, 31, replace=False)
        xi[m, pos] = rng.choice([-1, 1], size=31)
    x = S.bf16_bits(xi.astype(np.float32))
    y = gq.linear(bf16_dev(x), p)
    torch.cuda.synchronize()
    exact = (xi @ base.astype(np.int64).T) * 2.0 ** -6
    assert np.abs(exact).max() / 2 ** -6 < 256
    assert np.array_equal(O.bf16_bits_to_f64(y_bits(y)), exact)


@pytest.mark.parametrize("M", [2, 40, 200])
def test_linear_matches_torch_on_dequantized(M):
    """gq_linear against torch.matmul on the library's own fp32 dequant: the
    same math up to fp32 accumulation order and the fp16 weight rounding."""
    N, K = 320, 1024
    W = S.decode_weight(2, N=N, K=K)
    p = gq.quantize_pack(to_dev(W), 4)
    xb = bf16_dev(S.activations(M, K, 3))
    y = gq.linear(xb, p).float()
    ref = xb.float() @ gq.dequant(p, torch.float32).T
    rel = (torch.linalg.norm(y - ref) / torch.linalg.norm(ref)).item()
    assert rel <= 2e-3


def test_empty_and_degenerate_calls():
    N, K = 128, 256
    p = gq.quantize_pack(to_dev(S.decode_weight(3, N=N, K=K)), 4)
    x = torch.zeros((0, K), dtype=torch.bfloat16, device="cuda")
    y = gq.linear(x, p)
    assert y.shape == (0, N)
    z = gq.quantize_pack(torch.zeros((0, K), dtype=torch.float32, device="cuda"), 4)
    assert z.N == 0
    torch.cuda.synchronize()


def test_repeat_is_bitwise_deterministic():
    N, K, M = 1024, 2048, 100
    p = gq.quantize_pack(to_dev(S.decode_weight(0, N=N, K=K)), [4, 2, 2, 4, 2, 2, 4, 2], 128)
    x = bf16_dev(S.activations(M, K, 9))
    a = y_bits(gq.linear(x, p))
    b = y_bits(gq.linear(x, p))
    assert np.array_equal(a, b)
    x1 = x[:3].contiguous()
    assert np.array_equal(y_bits(gq.linear(x1, p)), y_bits(gq.linear(x1, p)))


def test_one_workspace_across_paths():
    """Small-batch (split K), prefill and small-batch calls of two shapes
    reuse one workspace in turn; every result stays within the bar."""
    shapes = [(1024, 2048, [4]), (640, 4096, [2])]
    packs = []
    for N, K, bits in shapes:
        W = S.decode_weight(2, N=N, K=K)
        ref = O.quantize_pack(W, O.Layout(K, N, N, bits))
        packs.append((K, ref, upload_packed(ref)))
    need = max(gq.gq_linear_workspace_bytes(p.layout, M) for _, _, p in packs for M in (12, 24, 80))
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for M in (12, 80, 24, 12):
        for K, ref, p in packs:
            x = S.activations(M, K, 40 + M)
            y = gq.linear(bf16_dev(x), p, ws=ws)
            torch.cuda.synchronize()
            linear_gate(y_bits(y), O.linear(x, ref), x, ref)
