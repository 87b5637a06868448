"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one gq_quantize_pack / gq_linear call per linear).

Packed codes, scales and zeros are compared byte for byte over whole layers.
Decode outputs (M <= 32) are compared in full: normwise relative error <=
2e-3 plus the elementwise bound of test_gpu_parity.  The M = 2048 prefill
GEMM is checked at sampled (m, n) that hit every 256 x 256 output tile
(including the tiles of an incomplete last round, which are split along K).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

gq = pytest.importorskip("quantized_gemm_groupwise_amd")
from tests.gpu_util import bf16_dev, y_bits  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def _say(*a):
    print(*a, flush=True)


def sample_rows(N, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(n, N), replace=False).tolist())
    rows |= {0, N - 1}
    return sorted(rows)


def oracle_packed_rows(W, block_n, bits, rows):
    """Oracle packing of just `rows` (a layout of len(rows) uniform rows per
    block width), with a map row -> position."""
    out = {}
    K = W.shape[1]
    for r in rows:
        b = bits[r // block_n]
        p = O.quantize_pack(W[r:r + 1], O.Layout(K, 1, 1, [b]))
        out[r] = p
    return out


def check_linear_sample(y, x_bits, W, block_n, bits, rows, ms):
    yb = y_bits(y)
    refs = oracle_packed_rows(W, block_n, bits, rows)
    y_ref = np.zeros((len(ms), len(rows)))
    bound_w = np.zeros((len(ms), len(rows)))
    xs = x_bits[ms]
    xa = np.abs(O.bf16_bits_to_f64(xs))
    for i, r in enumerate(rows):
        y_ref[:, i] = O.linear(xs, refs[r])[:, 0]
        bound_w[:, i] = xa @ np.abs(O.dequant(refs[r]).astype(np.float64))[0]
    yg = O.bf16_bits_to_f64(yb[np.ix_(ms, rows)])
    normwise = np.linalg.norm(yg - y_ref) / np.linalg.norm(y_ref)
    assert normwise <= 2e-3, normwise
    bound = 2.0 ** -8 * np.abs(y_ref) + 2.0 ** -10 * bound_w
    assert np.all(np.abs(yg - y_ref) <= bound), int((np.abs(yg - y_ref) > bound).sum())
    return normwise


def oracle_full(W, block_n, bits, chunk_blocks=16):
    """The oracle's packing of a whole layer, computed in runs of whole
    blocks (groups are independent, so the bytes are the same)."""
    N, K = W.shape
    L = O.Layout(K, N, block_n, list(bits))
    cb, ng, _ = L.sizes()
    codes = np.zeros(cb, np.uint8)
    scales = np.zeros(ng, np.uint16)
    zeros = np.zeros(ng, np.uint8)
    flags = 0
    blocks = list(L.blocks())
    step = chunk_blocks if block_n * chunk_blocks <= 4096 else 1
    for i in range(0, len(blocks), step):
        run = blocks[i:i + step]
        r0, r1 = run[0][1], run[-1][1] + block_n
        sub = O.quantize_pack(W[r0:r1], O.Layout(K, r1 - r0, block_n, [b[2] for b in run]))
        c0, g0 = run[0][4], run[0][5]
        codes[c0:c0 + sub.codes.size] = sub.codes
        scales[g0:g0 + sub.scales.size] = sub.scales
        zeros[g0:g0 + sub.zeros.size] = sub.zeros
        flags |= sub.flags
    return O.Packed(L, codes, scales, zeros, flags)


def check_packed_full(p, ref):
    cb, sb, zb = gq.gq_packed_bytes(p.layout)
    assert cb == ref.codes.size and sb == 2 * ref.scales.size and zb == ref.zeros.size
    assert np.array_equal(p.codes.cpu().numpy()[:cb], ref.codes), "codes differ"
    assert np.array_equal(p.scales.cpu().numpy().view(np.uint16)[: sb // 2], ref.scales), "scales differ"
    assert np.array_equal(p.zeros.cpu().numpy()[:zb], ref.zeros), "zeros differ"
    assert int(p.flags.cpu().item()) == ref.flags


def check_linear_full(y, x_bits, ref, wabs):
    """Every output against the fp64 oracle; wabs = |W_hat| in fp64."""
    y_ref = O.linear(x_bits, ref)
    yg = O.bf16_bits_to_f64(y_bits(y))
    normwise = np.linalg.norm(yg - y_ref) / np.linalg.norm(y_ref)
    assert normwise <= 2e-3, normwise
    bound = 2.0 ** -8 * np.abs(y_ref) + 2.0 ** -10 * (np.abs(O.bf16_bits_to_f64(x_bits)) @ wabs.T)
    bad = np.abs(yg - y_ref) > bound
    assert not bad.any(), f"{bad.sum()} outputs outside the bound"
    return normwise


def test_small_layer_config():
    """K = N = 512, INT4 g128, M = 4: full comparison."""
    d = S.small_layer()
    ref = O.quantize_pack(d["W"], O.Layout(512, 512, 512, [4]))
    p = gq.quantize_pack(torch.from_numpy(d["W"]).cuda(), 4)
    torch.cuda.synchronize()
    cb, sb, zb = gq.gq_packed_bytes(p.layout)
    assert np.array_equal(p.codes.cpu().numpy()[:cb], ref.codes)
    assert np.array_equal(p.scales.cpu().numpy().view(np.uint16)[: sb // 2], ref.scales)
    assert np.array_equal(p.zeros.cpu().numpy()[:zb], ref.zeros)
    y = gq.linear(bf16_dev(d["x"]), p)
    torch.cuda.synchronize()
    r = O.compare_linear(y_bits(y), O.linear(d["x"], ref))
    assert r["normwise"] <= 2e-3 and r["max_ulp"] <= 1


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("j", [0, 1, 2, 3])
def test_llama3_8b_decode_layers(j, bits):
    """Llama-3-8B-shaped layers, INT4 (M = 1) and INT2 (M in {1, 4, 16}):
    the whole packed layer byte for byte and every output."""
    N, K = S.LLAMA3_8B_SHAPE_LIST[j]
    W = S.decode_weight(j)
    _say("decode layer", j, N, K, "INT", bits)
    p = gq.quantize_pack(torch.from_numpy(W).cuda(), bits)
    torch.cuda.synchronize()
    ref = oracle_full(W, N, [bits])
    assert ref.flags == 0
    check_packed_full(p, ref)
    wabs = np.abs(O.dequant(ref)).astype(np.float64)
    for M in ((1,) if bits == 4 else (1, 4, 16)):
        x = S.decode_x(j, M)
        y = gq.linear(bf16_dev(x), p)
        torch.cuda.synchronize()
        _say("  M", M, "normwise", check_linear_full(y, x, ref, wabs))


# Layer-mix linears: 0 (q, INT2), 61 (up, INT2), 223 (down, INT2) and the
# INT4 linears 5 (up), 64 (k) and 69 (down) of the seeded assignment
@pytest.mark.parametrize("pick", [0, 61, 223, 5, 64, 69])
def test_layer_mix_linears(pick):
    """Linears of the 224-linear Layer-mix model at M in {1, 8, 32}, at their
    full shapes and the launch plans the benchmark uses: the packed linear
    byte for byte and every output."""
    assign = S.layer_mix_assignment()
    l, name, N, K, bits = assign[pick]
    idx = [n for (n, _, _) in S.LLAMA3_8B_LAYER].index(name)
    W = S.layer_mix_weight(l, idx, N, K)
    _say("layer-mix", pick, l, name, N, K, bits)
    p = gq.quantize_pack(torch.from_numpy(W).cuda(), bits)
    torch.cuda.synchronize()
    ref = oracle_full(W, N, [bits])
    check_packed_full(p, ref)
    wabs = np.abs(O.dequant(ref)).astype(np.float64)
    for M in (1, 8, 32):
        x = S.layer_mix_x(K, M)
        y = gq.linear(bf16_dev(x), p)
        torch.cuda.synchronize()
        _say("  M", M, "normwise", check_linear_full(y, x, ref, wabs))


def tile_sample(M, N, rng, per=2, tile=256):
    """(ms, rows): `per` rows of every 256-row band of m and `per` output
    channels of every 256-column band of n, so every (m, n) tile of the GEMM
    holds per^2 sampled outputs."""
    ms = sorted({int(t + rng.integers(min(tile, M - t))) for t in range(0, M, tile) for _ in range(per)}
                | {0, M - 1})
    rows = sorted({int(t + rng.integers(min(tile, N - t))) for t in range(0, N, tile) for _ in range(per)}
                  | {0, N - 1})
    return ms, rows


@pytest.mark.parametrize("j", [0, 1])
def test_channel_mix_prefill(j):
    """70B-class MLP, Channel-mix INT4/INT2 blocks of 128 channels, M = 2048."""
    N, K = S.MLP70B_SHAPES[j]
    W, bits = S.channel_mix_weight(j)
    _say("channel-mix", j, N, K, sum(b == 4 for b in bits), "INT4 blocks of", len(bits))
    p = gq.quantize_pack(torch.from_numpy(W).cuda(), bits, 128)
    torch.cuda.synchronize()
    ref = oracle_full(W, 128, bits)
    assert ref.flags == 0
    check_packed_full(p, ref)
    del ref
    x = S.channel_mix_x(j)
    y = gq.linear(bf16_dev(x), p)
    torch.cuda.synchronize()
    ms, rows = tile_sample(2048, N, np.random.default_rng(30 + j))
    _say("  sampled", len(ms), "x", len(rows), "outputs over every 256 x 256 tile")
    check_linear_sample(y, x, W, 128, bits, rows, ms)


@pytest.mark.parametrize("K,bits", [(4096, [4]), (8192, [4, 2] * 33)])
def test_gemm_tail_split(K, bits):
    """M = 2048, N = 8448: 264 tiles of 256 x 256, so the last 8 tiles (the
    columns 8192..8447) are cut along K (2 parts at K = 4096, 4 at 8192)
    and summed by the tail reduction."""
    M, N = 2048, 8448
    block_n = N if len(bits) == 1 else 128
    W = S.decode_weight(7, N=N, K=K)
    _say("gemm tail split", M, N, K, len(bits), "blocks")
    p = gq.quantize_pack(torch.from_numpy(W).cuda(), bits, block_n)
    torch.cuda.synchronize()
    rng = np.random.default_rng(70 + K)
    ms, rows = tile_sample(M, N, rng)
    rows = sorted(set(rows) | set((8192 + rng.choice(256, 20, replace=False)).tolist()))
    x = S.activations(M, K, 71)
    y = gq.linear(bf16_dev(x), p)
    torch.cuda.synchronize()
    check_linear_sample(y, x, W, block_n, bits, rows, ms)
