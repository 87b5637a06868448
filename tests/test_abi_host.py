"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/gq.h declares, sizes buffers like the oracle's layout,
and rejects bad arguments before anything is enqueued.

Pointer arguments in the error-path tests are fake addresses: every checked
error returns before any device memory is touched or any kernel launched.
"""
import ctypes
import os
import re

import pytest

import oracle as O

gq = pytest.importorskip("quantized_gemm_groupwise_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return gq.load_library()


def test_exports_match_header(lib):
    hdr = open(os.path.join(ROOT, "include", "gq.h")).read()
    declared = set(re.findall(r"^\S.*?\b(gq_[a-z_]+)\s*\(", hdr, flags=re.M))
    assert declared == set(gq.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_single_hip_runtime_mapped(lib):
    maps = {l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l}
    assert len(maps) == 1, maps


@pytest.mark.parametrize("K,N,block_n,bits", [
    (512, 512, 512, [4]), (4096, 14336, 14336, [4]), (14336, 4096, 4096, [2]),
    (8192, 28672, 128, [4, 2] * 112), (256, 384, 128, [2, 4, 2]), (64, 5, 5, [2]),
    (4096, 4096, 4096, [8]), (1024, 640, 128, [8, 2, 4, 8, 2]), (128, 3, 3, [8]),
])
def test_packed_sizes_match_oracle_layout(K, N, block_n, bits):
    cb, sb, zb = gq.gq_packed_bytes(gq.make_layout(K, N, block_n, bits))
    ocb, ons, onz = O.Layout(K, N, block_n, bits).sizes()
    assert (cb, sb, zb) == (ocb, 2 * ons, onz)


def _st(f, *a):
    return f(*a)


def test_layout_validation(lib):
    P = gq.make_layout
    c, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    def pb(lay):
        return lib.gq_packed_bytes(ctypes.byref(lay), ctypes.byref(c), ctypes.byref(s), ctypes.byref(z))
    assert pb(P(512, 512, 512, [4])) == gq.GQ_OK
    assert pb(P(512, 512, 512, [3])) == gq.GQ_ERR_BITS
    assert pb(P(512, 512, 512, [16])) == gq.GQ_ERR_BITS
    assert pb(P(512, 512, 512, [8])) == gq.GQ_OK
    assert pb(P(192, 512, 512, [8])) == gq.GQ_ERR_SHAPE      # 8-bit groups are 128
    assert pb(P(192, 512, 512, [4])) == gq.GQ_ERR_SHAPE      # K % 128
    assert pb(P(192, 512, 512, [2])) == gq.GQ_OK              # K % 64 ok for INT2
    assert pb(P(100, 512, 512, [2])) == gq.GQ_ERR_SHAPE
    assert pb(P(0, 512, 512, [4])) == gq.GQ_ERR_SHAPE
    assert pb(P(512, 500, 128, [4] * 4)) == gq.GQ_ERR_SHAPE   # N % block_n
    assert pb(P(512, 256, 64, [4] * 4)) == gq.GQ_ERR_SHAPE    # multi-block needs 128 | block_n
    assert pb(P(512, 1025 * 128, 128, [4] * 1025)) == gq.GQ_ERR_SHAPE   # too many blocks
    assert pb(P(512, 0, 1, [])) == gq.GQ_OK
    assert lib.gq_packed_bytes(None, ctypes.byref(c), ctypes.byref(s), ctypes.byref(z)) == gq.GQ_ERR_NULL_ARG
    lay = gq.gq_layout(512, 512, 512, None)
    assert pb(lay) == gq.GQ_ERR_NULL_ARG


def test_argument_errors_before_launch(lib):
    lay = gq.make_layout(512, 256, 256, [4])
    A = 0x10000        # aligned fake address
    bad = 0x10008      # 8-byte aligned only
    Q = lambda *a: lib.gq_quantize_pack(ctypes.byref(lay), *a)
    assert Q(None, A, A, A, None, None) == gq.GQ_ERR_NULL_ARG
    assert Q(bad, A, A, A, None, None) == gq.GQ_ERR_ALIGNMENT
    assert Q(A, bad, A, A, None, None) == gq.GQ_ERR_ALIGNMENT
    assert Q(A, A, A + 1, A, None, None) == gq.GQ_ERR_ALIGNMENT
    assert Q(A, A, None, A, None, None) == gq.GQ_ERR_NULL_ARG
    assert Q(A, A, A, A, A + 2, None) == gq.GQ_ERR_ALIGNMENT
    F = lambda *a: lib.gq_fake_quant(ctypes.byref(lay), *a)
    assert F(A, 7, A, None, None) == gq.GQ_ERR_DTYPE
    assert F(None, gq.GQ_BF16, A, None, None) == gq.GQ_ERR_NULL_ARG
    assert F(bad, gq.GQ_BF16, A, None, None) == gq.GQ_ERR_ALIGNMENT
    assert F(A, gq.GQ_FP32, None, None, None) == gq.GQ_ERR_NULL_ARG
    assert F(A, gq.GQ_FP32, bad, None, None) == gq.GQ_ERR_ALIGNMENT
    assert F(A, gq.GQ_FP32, A, A + 2, None) == gq.GQ_ERR_ALIGNMENT
    D = lambda *a: lib.gq_dequant(ctypes.byref(lay), *a)
    assert D(A, A, A, 7, A, None) == gq.GQ_ERR_DTYPE
    assert D(A, A, A, gq.GQ_FP32, bad, None) == gq.GQ_ERR_ALIGNMENT
    assert D(None, A, A, gq.GQ_FP32, A, None) == gq.GQ_ERR_NULL_ARG
    Lf = lambda M, act, x, y, ws, wsb: lib.gq_linear(ctypes.byref(lay), M, act, x, A, A, A, y, ws, wsb, None)
    assert Lf(-1, gq.GQ_BF16, A, A, None, 0) == gq.GQ_ERR_SHAPE
    assert Lf(1, gq.GQ_FP32, A, A, None, 0) == gq.GQ_ERR_DTYPE
    assert Lf(1, gq.GQ_BF16, bad, A, None, 0) == gq.GQ_ERR_ALIGNMENT
    assert Lf(1, gq.GQ_BF16, A, A + 1, None, 0) == gq.GQ_ERR_ALIGNMENT
    assert Lf(1, gq.GQ_BF16, A, None, None, 0) == gq.GQ_ERR_NULL_ARG
    need = gq.gq_linear_workspace_bytes(lay, 100)
    assert need > 0
    assert Lf(100, gq.GQ_BF16, A, A, None, 0) == gq.GQ_ERR_WORKSPACE
    assert Lf(100, gq.GQ_BF16, A, A, A, need - 1) == gq.GQ_ERR_WORKSPACE
    assert Lf(100, gq.GQ_BF16, A, A, A + 16, need) == gq.GQ_ERR_ALIGNMENT
    # empty work is a no-op that succeeds without touching any pointer
    assert Lf(0, gq.GQ_BF16, None, None, None, 0) == gq.GQ_OK
    lay0 = gq.make_layout(512, 0, 1, [])
    assert lib.gq_quantize_pack(ctypes.byref(lay0), None, None, None, None, None, None) == gq.GQ_OK
    assert lib.gq_fake_quant(ctypes.byref(lay0), None, gq.GQ_BF16, None, None, None) == gq.GQ_OK


def test_dx_argument_errors_before_launch(lib):
    """gq_linear_dx: every refusal happens on the host, before a launch."""
    lay = gq.make_layout(512, 256, 128, [4, 2])
    A, bad = 0x10000, 0x10008
    Dx = lambda M, act, dy, dx, ws, wsb: lib.gq_linear_dx(ctypes.byref(lay), M, act, dy, A, A, A, dx,
                                                          ws, wsb, None)
    assert Dx(-1, gq.GQ_BF16, A, A, None, 0) == gq.GQ_ERR_SHAPE
    assert Dx(1, gq.GQ_FP32, A, A, None, 0) == gq.GQ_ERR_DTYPE
    assert Dx(1, gq.GQ_BF16, bad, A, None, 0) == gq.GQ_ERR_ALIGNMENT
    assert Dx(1, gq.GQ_BF16, None, A, None, 0) == gq.GQ_ERR_NULL_ARG
    assert Dx(1, gq.GQ_BF16, A, A + 1, None, 0) == gq.GQ_ERR_ALIGNMENT
    assert Dx(1, gq.GQ_BF16, A, None, None, 0) == gq.GQ_ERR_NULL_ARG
    need = gq.gq_linear_dx_workspace_bytes(lay, 300)
    # dY as fp16 padded to whole 256 x 256 tiles, plus the row exponents
    assert need >= 512 * 256 * 2 + 300 * 4 and need % 256 == 0
    assert Dx(300, gq.GQ_BF16, A, A, None, 0) == gq.GQ_ERR_WORKSPACE
    assert Dx(300, gq.GQ_BF16, A, A, A, need - 1) == gq.GQ_ERR_WORKSPACE
    assert Dx(300, gq.GQ_BF16, A, A, A + 16, need) == gq.GQ_ERR_ALIGNMENT
    assert Dx(0, gq.GQ_BF16, None, None, None, 0) == gq.GQ_OK
    # N % 8 != 0: refused by both calls
    odd = gq.make_layout(512, 12, 12, [4])
    with pytest.raises(gq.GqError):
        gq.gq_linear_dx_workspace_bytes(odd, 4)
    assert lib.gq_linear_dx(ctypes.byref(odd), 4, gq.GQ_BF16, A, A, A, A, A, A, 1 << 20, None) \
        == gq.GQ_ERR_SHAPE
    # a small tile grid splits the n range: fp32 parts in the workspace
    wide = gq.make_layout(256, 16384, 16384, [4])
    assert gq.gq_linear_dx_workspace_bytes(wide, 64) >= 2 * 64 * 256 * 4


def test_kv_attention_argument_errors_before_launch(lib):
    """gq_kv_attention: shape, width and pointer checks on the host."""
    A, bad = 0x10000, 0x10008
    def cache(**kw):
        f = dict(batch=1, q_heads=32, kv_heads=8, head_dim=128, bits=4, t_packed=100, t_window=8,
                 k_codes=A, k_scales=A, k_zeros=A, v_codes=A, v_scales=A, v_zeros=A, k_window=A, v_window=A)
        f.update(kw)
        return gq.gq_kv_cache(*[f[n] for n, _ in gq.gq_kv_cache._fields_])
    KV = lambda c, q, o, ws, wsb: lib.gq_kv_attention(ctypes.byref(c), q, o, ws, wsb, None)
    need = gq.gq_kv_attention_workspace_bytes(cache())
    assert need > 0 and need % 256 == 0
    assert KV(cache(head_dim=64), A, A, A, need) == gq.GQ_ERR_SHAPE
    assert KV(cache(q_heads=12), A, A, A, need) == gq.GQ_ERR_SHAPE           # 12 / 8 heads
    assert KV(cache(q_heads=48, kv_heads=3), A, A, A, need) == gq.GQ_ERR_SHAPE   # 16 per head
    assert KV(cache(bits=3), A, A, A, need) == gq.GQ_ERR_BITS
    assert KV(cache(t_packed=0, t_window=0), A, A, A, need) == gq.GQ_ERR_SHAPE
    assert KV(cache(t_window=1025), A, A, A, need) == gq.GQ_ERR_SHAPE
    assert KV(cache(), bad, A, A, need) == gq.GQ_ERR_ALIGNMENT
    assert KV(cache(), A, None, A, need) == gq.GQ_ERR_NULL_ARG
    assert KV(cache(k_codes=bad), A, A, A, need) == gq.GQ_ERR_ALIGNMENT
    assert KV(cache(v_zeros=None), A, A, A, need) == gq.GQ_ERR_NULL_ARG
    assert KV(cache(k_window=None), A, A, A, need) == gq.GQ_ERR_NULL_ARG
    assert KV(cache(), A, A, None, need) == gq.GQ_ERR_WORKSPACE
    assert KV(cache(), A, A, A, need - 1) == gq.GQ_ERR_WORKSPACE
    assert KV(cache(), A, A, A + 16, need) == gq.GQ_ERR_ALIGNMENT
    assert lib.gq_kv_attention(None, A, A, A, need, None) == gq.GQ_ERR_NULL_ARG


def test_workspace_sizes():
    lay = gq.make_layout(4096, 14336, 14336, [4])
    # dot-product path, and the small-batch path on a wide layer up to 16
    # rows (its whole k range fits one workgroup): no scratch
    for M in (0, 1, 4, 5, 16):
        assert gq.gq_linear_workspace_bytes(lay, M) == 0
    # GEMM path: fp16 activations padded to whole tiles, row exponents
    for M in (64, 2048):
        ws = gq.gq_linear_workspace_bytes(lay, M)
        assert ws >= M * 4096 * 2 + M * 4 and ws % 256 == 0
    # a narrow layer with a K range too long for one workgroup splits K
    # across workgroups: fp32 partials
    narrow = gq.make_layout(28672, 256, 256, [4])
    ws = gq.gq_linear_workspace_bytes(narrow, 8)
    assert ws >= 2 * 8 * 256 * 4 and ws % 256 == 0


def test_noalloc_refusals_before_launch(lib):
    """gq_linear_noalloc: the checks of gq_linear, then GQ_ERR_TOO_LARGE for a
    call whose workspace need exceeds the static scratch, all on the host."""
    lay = gq.make_layout(4096, 1024, 1024, [4])
    A, bad = 0x10000, 0x10008
    NA = lambda lay, M, act, x, y: lib.gq_linear_noalloc(ctypes.byref(lay), M, act, x, A, A, A, y, None)
    assert NA(lay, -1, gq.GQ_BF16, A, A) == gq.GQ_ERR_SHAPE
    assert NA(lay, 1, gq.GQ_FP32, A, A) == gq.GQ_ERR_DTYPE
    assert NA(lay, 1, gq.GQ_BF16, bad, A) == gq.GQ_ERR_ALIGNMENT
    assert NA(lay, 1, gq.GQ_BF16, A, None) == gq.GQ_ERR_NULL_ARG
    assert NA(lay, 0, gq.GQ_BF16, None, None) == gq.GQ_OK
    big = gq.make_layout(28672, 8192, 8192, [2])
    assert gq.gq_linear_workspace_bytes(big, 2048) > gq.GQ_NOALLOC_SCRATCH_BYTES
    assert NA(big, 2048, gq.GQ_BF16, A, A) == gq.GQ_ERR_TOO_LARGE


def test_group_plan_refusals_and_size(lib):
    """Grouped decode plans: argument checks on the host, the plan size, and a
    refused launch of anything that is not a plan."""
    A, bad = 0x10000, 0x10008
    lay = gq.make_layout(4096, 1024, 1024, [4])
    mix = gq.make_layout(1024, 384, 128, [4, 2, 4])
    it = lambda l, x=A, c=A, y=A: gq.gq_group_item(l, x, c, A, A, y)
    items = [it(lay), it(mix)]
    n = gq.gq_group_plan_bytes(items, 1)
    # header, two records, one int32 per workgroup of 8 rows
    assert n > (1024 // 8 + 384 // 8) * 4
    assert gq.gq_group_plan_bytes(items, 4) == n
    for M in (0, 5):
        with pytest.raises(gq.GqError):
            gq.gq_group_plan_bytes(items, M)
    with pytest.raises(gq.GqError):
        gq.gq_group_plan_bytes(items, 1, gq.GQ_FP32)
    for bad_item in (it(lay, x=bad), it(lay, c=bad), it(lay, y=A + 1), it(lay, x=None),
                     it(gq.make_layout(100, 1024, 1024, [4]))):
        with pytest.raises(gq.GqError):
            gq.gq_group_plan_bytes([it(lay), bad_item], 1)
    buf = ctypes.create_string_buffer(n)
    assert gq.gq_group_plan(items, 1, gq.GQ_BF16, buf, n - 1) == gq.GQ_ERR_WORKSPACE
    assert gq.gq_group_plan(items, 1, gq.GQ_BF16, buf, n) == gq.GQ_OK
    # the launch refuses a misaligned device copy and anything not a plan
    assert lib.gq_linear_group(buf, bad, None) == gq.GQ_ERR_ALIGNMENT
    junk = ctypes.create_string_buffer(n)
    assert lib.gq_linear_group(junk, A, None) == gq.GQ_ERR_SHAPE
    assert lib.gq_linear_group(None, A, None) == gq.GQ_ERR_NULL_ARG
    # a group of empty linears needs no launch
    empty = gq.make_layout(512, 0, 1, [])
    n0 = gq.gq_group_plan_bytes([it(empty, x=None, c=None, y=None)], 1)
    b0 = ctypes.create_string_buffer(n0)
    assert gq.gq_group_plan([it(empty, x=None, c=None, y=None)], 1, gq.GQ_BF16, b0, n0) == gq.GQ_OK
    assert lib.gq_linear_group(b0, A, None) == gq.GQ_OK


def test_eight_bit_paths_refused_before_launch(lib):
    """Layouts with 8-bit blocks run quantize/pack, dequant, fake quant, the
    M <= 4 decode kernel and grouped decode; the other matmul paths refuse
    them with GQ_ERR_UNSUPPORTED on the host, before any launch."""
    A = 0x10000
    for lay in (gq.make_layout(1024, 256, 256, [8]), gq.make_layout(1024, 384, 128, [4, 8, 2])):
        assert gq.gq_linear_workspace_bytes(lay, 4) == 0
        for M in (5, 32, 2048):
            with pytest.raises(gq.GqError) as e:
                gq.gq_linear_workspace_bytes(lay, M)
            assert e.value.status == gq.GQ_ERR_UNSUPPORTED
            assert lib.gq_linear(ctypes.byref(lay), M, gq.GQ_BF16, A, A, A, A, A, A, 1 << 30,
                                 None) == gq.GQ_ERR_UNSUPPORTED
            assert lib.gq_linear_noalloc(ctypes.byref(lay), M, gq.GQ_BF16, A, A, A, A, A,
                                         None) == gq.GQ_ERR_UNSUPPORTED
        sz = ctypes.c_size_t()
        assert lib.gq_linear_dx_workspace_bytes(ctypes.byref(lay), 8, gq.GQ_BF16,
                                                ctypes.byref(sz)) == gq.GQ_ERR_UNSUPPORTED
        assert lib.gq_linear_dx(ctypes.byref(lay), 8, gq.GQ_BF16, A, A, A, A, A, A, 1 << 30,
                                None) == gq.GQ_ERR_UNSUPPORTED
        # grouped decode plans accept them
        n = gq.gq_group_plan_bytes([gq.gq_group_item(lay, A, A, A, A, A)], 4)
        assert n > 0


def test_status_strings():
    for st in range(10):
        assert gq.gq_status_string(st).startswith("GQ_")
    assert "unknown" in gq.gq_status_string(99)


def test_product_path_refuses_missing_library(tmp_path):
    import importlib
    mod = importlib.import_module("quantized_gemm_groupwise_amd")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            mod.load_library(str(tmp_path / "nope.so"))
    finally:
        mod._lib = saved


def test_stream_probe_library_refuses_bad_arguments():
    """The benchmark's streaming-read probe (its own library) loads and
    refuses a null buffer or sink, a zero or unaligned size and an unaligned
    address before any launch."""
    import torch  # noqa: F401  -- torch's HIP runtime first, as for libgq
    path = os.path.join(ROOT, "quantized_gemm_groupwise_amd", "libgq_probe.so")
    probe = ctypes.CDLL(path)
    fn = probe.gqprobe_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    buf, sink = 0x7F0000000000, 0x7F0000100000
    assert fn(None, 1024, sink, None) == -1
    assert fn(buf, 1024, None, None) == -1
    assert fn(buf, 0, sink, None) == -1
    assert fn(buf, 1000, sink, None) == -1
    assert fn(buf + 8, 1024, sink, None) == -1
