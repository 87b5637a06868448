"""GPU parity of 8-bit entries in the bit map (blocks kept at higher precision
inside a low-bit model, as section 4.2 of '大模型量化实战' keeps lm_head at 8
bits; q_max 255, groups of 128): the HIP library against the CPU oracle.

Bar, as for INT4 / INT2: packed codes, scales, zeros and flags byte-identical;
dequantized and fake-quantized weights bit-identical; decode-kernel outputs
within the normwise relative error 2e-3 of the fp64 oracle and the
elementwise bound 2^-8 |y_ref| + 2^-10 sum_k |x_k| |w_hat_k|; an exact-integer
case bit-exact; grouped decode bit-identical to gq_linear.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

gq = pytest.importorskip("quantized_gemm_groupwise_amd")
from tests.gpu_util import bf16_dev, gpu_quantize, to_dev, upload_packed, y_bits  # noqa: E402
from tests.test_gpu_parity import _fq_bytes, assert_packed_equal, linear_gate  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------- quantize

@pytest.mark.parametrize("N,K,block_n,bits", [
    (1, 128, 1, [8]), (3, 640, 3, [8]), (130, 1152, 130, [8]), (256, 4096, 256, [8]),
    (384, 1024, 128, [8, 4, 2]), (512, 2048, 128, [2, 8, 8, 4]),
])
def test_quantize_int8_shapes(N, K, block_n, bits):
    W = S.decode_weight(5, N=N, K=K)
    _say("quantize int8", N, K, block_n, bits)
    assert_packed_equal(W, block_n, bits)


def test_quantize_int8_edge_groups():
    """Degenerate groups, the fp16 scale tie, subnormal and vanishing scales,
    exact ties, one-sided groups (zero point clamped to 0 and to 255), fp32
    denormals; then fp16 overflow and a non-finite group (its codes are
    unspecified, its flag is not)."""
    g, Q = 128, 255
    rows = [np.full(g, 0.37, np.float32), np.full(g, -2.6, np.float32)]
    r = np.zeros(g, np.float32); r[1] = Q * (1 + 2 ** -11); rows.append(r)      # scale tie
    r = np.zeros(g, np.float32); r[1] = Q * 3 * 2 ** -26; rows.append(r)        # subnormal scale
    r = np.zeros(g, np.float32); r[1] = Q * 2.0 ** -25; rows.append(r)          # scale -> 0 -> 1
    r = (np.arange(g, dtype=np.float32) - 40.5) * np.float32(2 ** -7); rows.append(r)
    rows.append(np.linspace(3.0, 4.0, g, dtype=np.float32))                     # z clamps to 0
    rows.append(np.linspace(-4.0, -3.0, g, dtype=np.float32))                   # z clamps to 255
    r = np.zeros(g, np.float32); r[3] = 1e-39; r[4] = -3e-40; rows.append(r)
    W = np.stack(rows)
    _say("quantize int8 edge groups")
    ref = assert_packed_equal(W, W.shape[0], [8])
    assert ref.flags == O.FLAG_ZERO_CLAMPED
    W2 = np.stack([W[0], W[2]])
    W2[1, 7] = Q * 65520.0                                        # fp16 overflow
    ref = assert_packed_equal(W2, 2, [8])
    assert ref.flags == O.FLAG_SCALE_OVERFLOW
    W3 = np.stack([W[5], W[6]])
    W3[1, 9] = np.nan
    ref = O.quantize_pack(W3, O.Layout(g, 2, 2, [8]))
    codes, scales, zeros, flags, _ = gpu_quantize(W3, 2, [8])
    # row 1 is one-sided but non-finite: only its non-finite flag is reported
    assert flags == O.FLAG_NONFINITE == ref.flags
    assert np.array_equal(codes[:g], ref.codes[:g]) and scales[0] == ref.scales[0] and zeros[0] == ref.zeros[0]


# ------------------------------------------------- dequant and fake quant

@pytest.mark.parametrize("N,K,block_n,bits", [(256, 512, 256, [8]), (384, 1024, 128, [8, 2, 4])])
def test_dequant_int8_bit_exact(N, K, block_n, bits):
    W = S.decode_weight(2, N=N, K=K)
    ref = O.quantize_pack(W, O.Layout(K, N, block_n, bits))
    p = upload_packed(ref)
    for dt, name in [(torch.float32, "fp32"), (torch.float16, "fp16"), (torch.bfloat16, "bf16")]:
        out = gq.dequant(p, dt)
        torch.cuda.synchronize()
        exp = np.ascontiguousarray(O.dequant_as(ref, name)).view(np.uint8)
        assert np.array_equal(_fq_bytes(out, name), exp), name


@pytest.mark.parametrize("N,K,block_n,bits", [(3, 640, 3, [8]), (512, 1024, 128, [8, 4, 2, 8])])
def test_fake_quant_int8_bit_exact(N, K, block_n, bits):
    W = S.decode_weight(4, N=N, K=K)
    L = O.Layout(K, N, block_n, bits)
    w = to_dev(W)
    for dt, name in [(torch.float32, "fp32"), (torch.float16, "fp16"), (torch.bfloat16, "bf16")]:
        out = gq.fake_quant(w, bits, block_n, dt)
        torch.cuda.synchronize()
        assert np.array_equal(_fq_bytes(out, name), np.ascontiguousarray(O.fake_quant(W, L, name)).view(np.uint8)), name


# ------------------------------------------------------- decode matmul

@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("N,K,block_n,bits", [
    (512, 1024, 512, [8]),            # one 1 KB slice per row
    (300, 2048, 300, [8]),            # two slices: one load group
    (640, 4096, 640, [8]),            # rows streamed in load groups
    (129, 128, 129, [8]),             # short rows, ragged N
    (384, 1024, 128, [8, 4, 2]),      # Channel-mix with 8-bit blocks
    (256, 4096, 128, [4, 8]),         # the same, streamed rows
])
def test_linear_int8_gemv(M, N, K, block_n, bits):
    W = S.decode_weight(6, N=N, K=K)
    ref = O.quantize_pack(W, O.Layout(K, N, block_n, bits))
    p = upload_packed(ref)
    x = S.activations(M, K, 91 + M)
    _say("gemv int8", M, N, K, bits)
    y = gq.linear(bf16_dev(x), p)
    torch.cuda.synchronize()
    linear_gate(y_bits(y), O.linear(x, ref), x, ref)


def test_linear_int8_fp16_activations():
    M, N, K = 3, 512, 2048
    W = S.decode_weight(7, N=N, K=K)
    ref = O.quantize_pack(W, O.Layout(K, N, 128, [8, 8, 4, 2]))
    p = upload_packed(ref)
    x16 = (np.random.default_rng(5).standard_normal((M, K))).astype(np.float16)
    y = gq.linear(to_dev(x16), p)
    torch.cuda.synchronize()
    yref = x16.astype(np.float64) @ O.dequant(ref).astype(np.float64).T
    yg = y.cpu().numpy().astype(np.float64)
    assert np.linalg.norm(yg - yref) / np.linalg.norm(yref) <= 2e-3
    bound = 2.0 ** -8 * np.abs(yref) + 2.0 ** -10 * (np.abs(x16.astype(np.float64)) @ np.abs(O.dequant(ref).astype(np.float64)).T)
    assert np.all(np.abs(yg - yref) <= bound)


@pytest.mark.parametrize("M", [1, 3])
def test_linear_int8_exact_integer_case(M):
    """Every group spans exactly 255 steps of 2^-6 (its first two weights
    -127 and 128 steps), so S = 2^-6, z = 127 and code = weight/S + 127 for
    all 256 levels; x in {-1, 0, 1} on 31 positions away from the two
    endpoint columns, and the other weights within +-4 steps, keep |y| / 2^-6
    below 256: every exact result is a bf16 value and the output must be
    bit-exact."""
    rng = np.random.default_rng(40 + M)
    N, K = 192, 1024
    base = rng.integers(-4, 5, size=(N, K)).astype(np.int64)
    base[:, 0::128] = -127
    base[:, 1::128] = 128
    W = (base * 2.0 ** -6).astype(np.float32)
    ref = O.quantize_pack(W, O.Layout(K, N, N, [8]))
    c, s, z, _, _ = O.block_fields(ref, 0)
    assert np.all(s.astype(np.float64) == 2.0 ** -6) and np.all(z == 127)
    assert np.array_equal(c.astype(np.int64), base + 127)
    p = upload_packed(ref)
    free = np.array([k for k in range(K) if k % 128 > 1])
    xi = np.zeros((M, K), dtype=np.int64)
    for m in range(M):
        pos = rng.choice(free, 31, replace=False)
        xi[m, pos] = rng.choice([-1, 1], size=31)
    x = S.bf16_bits(xi.astype(np.float32))
    y = gq.linear(bf16_dev(x), p)
    torch.cuda.synchronize()
    exact = (xi @ base.T) * 2.0 ** -6
    assert np.abs(exact).max() / 2 ** -6 < 256
    assert np.array_equal(O.bf16_bits_to_f64(y_bits(y)), exact)


def test_int8_lm_head_rows_sampled():
    """A vocabulary-sized 8-bit layer (16384 x 4096, the lm_head case of
    section 4.2): the GPU packs the whole matrix; sampled rows are
    byte-identical to the oracle's, and the decode output (M = 1) on them is
    within the bound."""
    N, K = 16384, 4096
    W = S.decode_weight(8, N=N, K=K)
    p = gq.quantize_pack(to_dev(W), 8)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(4), np.arange(N - 4, N),
                                     np.random.default_rng(3).choice(N, 56, replace=False)]))
    sub = O.quantize_pack(W[rows], O.Layout(K, len(rows), len(rows), [8]))
    codes = p.codes.view(N, K).cpu().numpy()[rows]
    scales = p.scales.view(N, K // 128).cpu().numpy().view(np.uint16)[rows]
    zeros = p.zeros.view(N, K // 128).cpu().numpy()[rows]
    assert np.array_equal(codes.reshape(-1), sub.codes)
    assert np.array_equal(scales.reshape(-1), sub.scales)
    assert np.array_equal(zeros.reshape(-1), sub.zeros)
    x = S.activations(1, K, 13)
    y = gq.linear(bf16_dev(x), p)
    torch.cuda.synchronize()
    linear_gate(y_bits(y)[:, rows], O.linear(x, sub), x, sub)


# ------------------------------------------------------- grouped decode

@pytest.mark.parametrize("M", [1, 3])
def test_group_decode_int8_equals_linear(M):
    specs = [(4096, 1024, 4096, [8]), (1024, 4096, 1024, [8]), (384, 2048, 128, [8, 4, 2]),
             (512, 1024, 512, [4]), (256, 4096, 128, [2, 8])]
    items = []
    for i, (N, K, bn, bits) in enumerate(specs):
        W = S.decode_weight(9 + i, N=N, K=K)
        p = gq.quantize_pack(to_dev(W), bits, bn)
        x = bf16_dev(S.activations(M, K, 200 + i))
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        items.append((x, p, y))
    plan = gq.group_plan(items)
    gq.linear_group(plan)
    torch.cuda.synchronize()
    for i, (x, p, y) in enumerate(items):
        ref = gq.linear(x, p)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"linear {i} {specs[i]}"


def test_int8_unsupported_paths_raise():
    """M > 4 and the data gradient have no 8-bit kernel: refused on the host."""
    W = S.decode_weight(1, N=256, K=512)
    p = gq.quantize_pack(to_dev(W), 8)
    x = bf16_dev(S.activations(8, 512, 3))
    with pytest.raises(gq.GqError) as e:
        gq.linear(x, p)
    assert e.value.status == gq.GQ_ERR_UNSUPPORTED
