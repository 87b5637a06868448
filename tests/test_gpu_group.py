"""Grouped decode launch (gq_group_plan / gq_linear_group) against
independent gq_linear calls and the CPU oracle.

The grouped kernels run the single-linear decode arithmetic per row tile
(same accumulation order, same reductions, same rounding), so every output
must equal the one gq_linear writes, bit for bit.  The oracle check bounds
the same outputs against the fp64 product of the dequantized weights, and
graph replays of the grouped launch must reproduce the eager bytes.  The
224-linear Layer-mix pass is checked against 224 independent calls, in the
grouped launch (M = 1) and in the captured per-linear pass the benchmark
times with one shared workspace (M = 1, 8, 32).
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


def _make(specs, M, seed, dtype=torch.bfloat16):
    """(x, packed, y, W, x_bits) per spec (N, K, bits, block_n); y starts as NaN."""
    out = []
    for i, (N, K, bits, block_n) in enumerate(specs):
        W = S.decode_weight(0, N=N, K=K, seed_base=seed + i)
        p = gq.quantize_pack(torch.from_numpy(W).cuda(), bits, block_n)
        xb = S.activations(M, K, seed + 500 + i)
        x = bf16_dev(xb)
        if dtype == torch.float16:
            xf = S.bf16_to_f32(xb).astype(np.float16)
            x = torch.from_numpy(xf.view(np.int16)).cuda().view(torch.float16)
            xb = xf.view(np.uint16)
        y = torch.full((M, N), float("nan"), dtype=dtype, device="cuda")
        out.append((x, p, y, W, xb))
    torch.cuda.synchronize()
    return out


SPECS = [
    (1024, 4096, [4], None),               # k/v-shaped, one load group per row
    (512, 14336, [2], None),               # long INT2 rows, streamed
    (256, 14336, [4], None),               # long INT4 rows, streamed
    (384, 1024, [4, 2, 4], 128),           # Channel-mix blocks
    (13, 192, [2], None),                  # ragged: 13 rows, K = 3 INT2 groups
    (100, 640, [4], None),                 # ragged: 100 rows (tile of 8 split)
    (8, 128, [4], None),                   # one tile, one INT4 group
]


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_group_equals_independent_calls(M):
    _say("group vs gq_linear, M =", M)
    items = _make(SPECS, M, 8100 + 10 * M)
    plan = gq.group_plan([(x, p, y) for (x, p, y, _, _) in items])
    gq.linear_group(plan)
    torch.cuda.synchronize()
    for i, (x, p, y, W, xb) in enumerate(items):
        ref = gq.linear(x, p)
        torch.cuda.synchronize()
        assert np.array_equal(y_bits(y), y_bits(ref)), f"item {i} {SPECS[i]}: differs from gq_linear"


SPECS_ALL_WIDTHS = [
    (256, 4096, [8], None),                # 8-bit rows of four slices, streamed
    (64, 1024, [8], None),                 # 8-bit, one slice
    (40, 2048, [8], None),                 # 8-bit, two slices (ragged tile)
    (384, 1024, [8, 4, 2], 128),           # Channel-mix with an 8-bit block
    (24, 512, [4], None),
    (100, 14336, [4], None),               # long INT4 rows next to short ones
    (16, 256, [2], None),
    (48, 8192, [2], None),
]


@pytest.mark.parametrize("M,dtype", [(1, torch.bfloat16), (3, torch.float16), (4, torch.bfloat16)])
def test_group_fused_launch_all_widths(M, dtype):
    """Several small classes of each width (8-bit, INT4, INT2), each run by
    one launch per width that holds all of that width's classes: every output
    is the bits gq_linear writes."""
    _say("fused classes, all widths, M =", M, dtype)
    items = _make(SPECS_ALL_WIDTHS, M, 8700 + M, dtype=dtype)
    plan = gq.group_plan([(x, p, y) for (x, p, y, _, _) in items])
    gq.linear_group(plan)
    torch.cuda.synchronize()
    for i, (x, p, y, W, xb) in enumerate(items):
        ref = gq.linear(x, p)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"item {i} {SPECS_ALL_WIDTHS[i]}"


@pytest.mark.parametrize("M", [3, 4])
def test_group_int2_full_size_m3_m4_equals_gq_linear(M):
    """INT2 rows run four per wave in the grouped kernels and at most two in
    gq_linear, so at M = 3 and 4 a wave reduces 16 values against 8.  A
    value's total must come out the same bits either way: the wave reduction
    adds the same lanes in the same tree for every number of values.  A
    different tree changes a bf16 output only near a rounding boundary, so
    this runs on full-size layers (up/gate and down, 18432 rows)."""
    _say("INT2 full size, grouped vs gq_linear, M =", M)
    specs = [(14336, 4096, [2], None), (4096, 14336, [2], None)]
    items = _make(specs, M, 9100 + M)
    plan = gq.group_plan([(x, p, y) for (x, p, y, _, _) in items])
    gq.linear_group(plan)
    torch.cuda.synchronize()
    for i, (x, p, y, W, xb) in enumerate(items):
        ref = gq.linear(x, p)
        torch.cuda.synchronize()
        d = int((y.view(torch.int16) != ref.view(torch.int16)).sum().item())
        assert d == 0, f"{specs[i]}: {d} outputs differ from gq_linear"


def test_group_fp16_activations():
    items = _make(SPECS[:4], 2, 8300, dtype=torch.float16)
    plan = gq.group_plan([(x, p, y) for (x, p, y, _, _) in items])
    gq.linear_group(plan)
    torch.cuda.synchronize()
    for i, (x, p, y, W, xb) in enumerate(items):
        ref = gq.linear(x, p)
        torch.cuda.synchronize()
        assert np.array_equal(y.view(torch.int16).cpu().numpy(), ref.view(torch.int16).cpu().numpy()), i


def test_group_against_oracle():
    """Every output of a small mixed group within the matmul tolerance of the
    fp64 oracle (normwise <= 2e-3, elementwise bf16-rounding bound)."""
    specs = [(64, 512, [4], None), (40, 256, [2], None), (256, 512, [2, 4], 128), (9, 128, [4], None)]
    items = _make(specs, 3, 8400)
    plan = gq.group_plan([(x, p, y) for (x, p, y, _, _) in items])
    gq.linear_group(plan)
    torch.cuda.synchronize()
    for (N, K, bits, block_n), (x, p, y, W, xb) in zip(specs, items):
        op = O.quantize_pack(W, O.Layout(K, N, N if block_n is None else block_n, bits))
        y_ref = O.linear(xb, op)
        yg = O.bf16_bits_to_f64(y_bits(y))
        assert np.linalg.norm(yg - y_ref) / np.linalg.norm(y_ref) <= 2e-3
        bound = 2.0 ** -8 * np.abs(y_ref) + 2.0 ** -10 * (np.abs(O.bf16_bits_to_f64(xb))
                                                          @ np.abs(O.dequant(op).astype(np.float64)).T)
        assert np.all(np.abs(yg - y_ref) <= bound)


@pytest.mark.parametrize("bits", [4, 2])
def test_group_llama3_8b_decode_step(bits):
    """The four Llama-3-8B decode linears (full size, M = 1) in one grouped
    call, equal to four gq_linear calls; sampled outputs against the oracle."""
    items = []
    for j, (N, K) in enumerate(S.LLAMA3_8B_SHAPE_LIST):
        W = S.decode_weight(j)
        p = gq.quantize_pack(torch.from_numpy(W).cuda(), bits)
        xb = S.decode_x(j, 1)
        y = torch.full((1, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        items.append((bf16_dev(xb), p, y, W, xb))
    plan = gq.group_plan([(x, p, y) for (x, p, y, _, _) in items])
    _say("decode step INT", bits, "classes", plan_classes(plan))
    gq.linear_group(plan)
    torch.cuda.synchronize()
    for j, (x, p, y, W, xb) in enumerate(items):
        ref = gq.linear(x, p)
        torch.cuda.synchronize()
        assert np.array_equal(y_bits(y), y_bits(ref)), f"linear {j}"
        N, K = S.LLAMA3_8B_SHAPE_LIST[j]
        rows = sorted(set(np.random.default_rng(40 + j).choice(N, 16, replace=False).tolist()) | {0, N - 1})
        op = O.quantize_pack(W[rows], O.Layout(K, len(rows), len(rows), [bits]))
        y_ref = O.linear(xb, op)[0]
        yg = O.bf16_bits_to_f64(y_bits(y)[0, rows])
        # per-element bound on the sample (a normwise statistic over a few
        # samples is noise): bf16 output rounding plus fp32 accumulation
        bound = 2.0 ** -8 * np.abs(y_ref) + 2.0 ** -10 * (np.abs(O.bf16_bits_to_f64(xb))
                                                          @ np.abs(O.dequant(op).astype(np.float64)).T)[0]
        assert np.all(np.abs(yg - y_ref) <= bound), f"linear {j}"


def plan_classes(plan):
    """Kernel classes of a plan (the header's class count)."""
    h = bytes(plan.host.raw[:64])
    return int.from_bytes(h[28:32], "little")


def test_group_graph_replays():
    """A captured grouped launch replayed several times, with eager work and
    synchronizations in between, reproduces the eager outputs every time."""
    items = _make(SPECS[:5], 1, 8500)
    plan = gq.group_plan([(x, p, y) for (x, p, y, _, _) in items])
    gq.linear_group(plan)
    torch.cuda.synchronize()
    eager = [y_bits(y).copy() for (_, _, y, _, _) in items]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        gq.linear_group(plan, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        gq.linear_group(plan)
    for rep in range(4):
        for (_, _, y, _, _) in items:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (_, _, y, _, _) in enumerate(items):
            assert np.array_equal(y_bits(y), eager[i]), f"replay {rep} item {i}"


def _layer_mix_packs():
    """The 224 Layer-mix linears packed on the GPU from weights drawn on the
    GPU (normal, sigma 0.02, 0.5% of input channels x20, the decode recipe);
    the comparison is between two GPU paths on the same packed bytes."""
    assign = S.layer_mix_assignment()
    gen = torch.Generator(device="cuda")
    packs = []
    for i, (l, name, N, K, bits) in enumerate(assign):
        gen.manual_seed(4000 + i)
        W = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02
        idx = torch.randperm(K, generator=gen, device="cuda")[: int(round(0.005 * K))]
        W[:, idx] *= 20.0
        packs.append(gq.quantize_pack(W, bits))
        del W
    torch.cuda.synchronize()
    return assign, packs


@pytest.fixture(scope="module")
def layer_mix():
    a, p = _layer_mix_packs()
    yield a, p
    del p
    torch.cuda.empty_cache()


def test_layer_mix_pass_grouped_equals_224_calls(layer_mix):
    assign, packs = layer_mix
    M = 1
    xs = {K: bf16_dev(S.layer_mix_x(K, M)) for K in (4096, 14336)}
    ys = [torch.full((M, p.N), float("nan"), dtype=torch.bfloat16, device="cuda") for p in packs]
    plan = gq.group_plan([(xs[p.K], p, y) for p, y in zip(packs, ys)])
    _say("layer-mix grouped: classes", plan_classes(plan))
    gq.linear_group(plan)
    torch.cuda.synchronize()
    for i, (p, y) in enumerate(zip(packs, ys)):
        ref = gq.linear(xs[p.K], p)
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"linear {i} {assign[i]}"


@pytest.mark.parametrize("M", [1, 8, 32])
def test_layer_mix_pass_graph_equals_224_calls(layer_mix, M):
    """The per-linear pass as the benchmark captures it (one HIP graph of 224
    gq_linear calls sharing one workspace) equals 224 independent eager
    calls, each with its own workspace."""
    assign, packs = layer_mix
    xs = {K: bf16_dev(S.layer_mix_x(K, M)) for K in (4096, 14336)}
    ys = [torch.full((M, p.N), float("nan"), dtype=torch.bfloat16, device="cuda") for p in packs]
    ws = torch.empty(max(gq.gq_linear_workspace_bytes(p.layout, M) for p in packs) + 256,
                     dtype=torch.uint8, device="cuda")

    def one_pass():
        for p, y in zip(packs, ys):
            gq.linear(xs[p.K], p, out=y, ws=ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        one_pass()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_pass()
    for y in ys:
        y.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for i, (p, y) in enumerate(zip(packs, ys)):
        own = torch.empty(max(gq.gq_linear_workspace_bytes(p.layout, M), 256), dtype=torch.uint8,
                          device="cuda")
        ref = gq.linear(xs[p.K], p, ws=own)
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"M={M} linear {i} {assign[i]}"
