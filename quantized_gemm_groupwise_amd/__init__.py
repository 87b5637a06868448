"""Python binding of libgq: group-wise INT4/INT2 quantization and the
weight-only low-bit matmul on AMD Instinct MI355X (gfx950).

The functions named gq_* mirror the C ABI in include/gq.h one to one and only
marshal arguments: every step of the computation runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.

Convenience layer:
    packed = quantize_pack(w, bits, block_n=None)   # w: fp32 cuda [N][K]
    y = linear(x, packed)                           # x: bf16/fp16 cuda [M][K]
    dx = linear_dx(dy, packed)                      # dy: bf16/fp16 cuda [M][N]
    w_hat = dequant(packed, torch.float32)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # noqa: F401  -- load torch's HIP runtime before libgq

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgq.so")

GQ_OK, GQ_ERR_NULL_ARG, GQ_ERR_SHAPE, GQ_ERR_BITS, GQ_ERR_ALIGNMENT, GQ_ERR_DTYPE, \
    GQ_ERR_WORKSPACE, GQ_ERR_HIP, GQ_ERR_TOO_LARGE, GQ_ERR_UNSUPPORTED = range(10)
GQ_NOALLOC_SCRATCH_BYTES = 64 << 20
GQ_BF16, GQ_FP16, GQ_FP32 = 0, 1, 2
GQ_FLAG_NONFINITE = 1
GQ_FLAG_SCALE_OVERFLOW = 2
GQ_FLAG_ZERO_CLAMPED = 4
GQ_MAX_BLOCKS = 1024
GROUP = {4: 128, 2: 64}

# Every symbol include/gq.h declares.
EXPORTS = ("gq_packed_bytes", "gq_quantize_pack", "gq_fake_quant", "gq_dequant",
           "gq_linear_workspace_bytes", "gq_linear", "gq_linear_noalloc", "gq_linear_dx_workspace_bytes",
           "gq_linear_dx", "gq_group_plan_bytes", "gq_group_plan", "gq_linear_group",
           "gq_kv_attention_workspace_bytes", "gq_kv_attention", "gq_status_string")


class GqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {gq_status_string(status)}")
        self.status = status


class gq_layout(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("N", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("bits", ctypes.POINTER(ctypes.c_uint8))]


class gq_group_item(ctypes.Structure):
    _fields_ = [("layout", gq_layout), ("x", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class gq_kv_cache(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("bits", ctypes.c_int32), ("t_packed", ctypes.c_int32),
                ("t_window", ctypes.c_int32),
                ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p), ("k_zeros", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p), ("v_zeros", ctypes.c_void_p),
                ("k_window", ctypes.c_void_p), ("v_window", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgq.so (built by quantized_gemm_groupwise_amd._build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m quantized_gemm_groupwise_amd._build`")
    lib = ctypes.CDLL(path)
    P, S, I32, VP = ctypes.POINTER, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p
    L = P(gq_layout)
    sig = {
        "gq_packed_bytes": ([L, P(S), P(S), P(S)], ctypes.c_int),
        "gq_quantize_pack": ([L, VP, VP, VP, VP, VP, VP], ctypes.c_int),
        "gq_fake_quant": ([L, VP, ctypes.c_int, VP, VP, VP], ctypes.c_int),
        "gq_dequant": ([L, VP, VP, VP, ctypes.c_int, VP, VP], ctypes.c_int),
        "gq_linear_workspace_bytes": ([L, I32, ctypes.c_int, P(S)], ctypes.c_int),
        "gq_linear": ([L, I32, ctypes.c_int, VP, VP, VP, VP, VP, VP, S, VP], ctypes.c_int),
        "gq_linear_noalloc": ([L, I32, ctypes.c_int, VP, VP, VP, VP, VP, VP], ctypes.c_int),
        "gq_linear_dx_workspace_bytes": ([L, I32, ctypes.c_int, P(S)], ctypes.c_int),
        "gq_linear_dx": ([L, I32, ctypes.c_int, VP, VP, VP, VP, VP, VP, S, VP], ctypes.c_int),
        "gq_group_plan_bytes": ([I32, P(gq_group_item), I32, ctypes.c_int, P(S)], ctypes.c_int),
        "gq_group_plan": ([I32, P(gq_group_item), I32, ctypes.c_int, VP, S], ctypes.c_int),
        "gq_linear_group": ([VP, VP, VP], ctypes.c_int),
        "gq_kv_attention_workspace_bytes": ([P(gq_kv_cache), P(S)], ctypes.c_int),
        "gq_kv_attention": ([P(gq_kv_cache), VP, VP, VP, S, VP], ctypes.c_int),
        "gq_status_string": ([ctypes.c_int], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def make_layout(K: int, N: int, block_n: int, bits) -> gq_layout:
    """A gq_layout over a host copy of `bits`.  The C side reads N / block_n
    entries, so a shorter list is refused here (it would be read past its
    end)."""
    if int(block_n) > 0 and int(N) >= 0 and int(N) % int(block_n) == 0 and len(bits) < int(N) // int(block_n):
        raise ValueError(f"bits needs N / block_n = {int(N) // int(block_n)} entries, got {len(bits)}")
    arr = (ctypes.c_uint8 * max(1, len(bits)))(*[int(b) for b in bits])
    lay = gq_layout(int(K), int(N), int(block_n), ctypes.cast(arr, ctypes.POINTER(ctypes.c_uint8)))
    lay._keep = arr  # keep the host array alive with the struct
    return lay


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------ one-to-one ABI wrappers

def gq_status_string(status: int) -> str:
    return load_library().gq_status_string(int(status)).decode()


def gq_packed_bytes(layout: gq_layout):
    c, s, z = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    st = load_library().gq_packed_bytes(ctypes.byref(layout), ctypes.byref(c), ctypes.byref(s),
                                        ctypes.byref(z))
    if st != GQ_OK:
        raise GqError(st, "gq_packed_bytes")
    return c.value, s.value, z.value


def gq_quantize_pack(layout, w_ptr, codes_ptr, scales_ptr, zeros_ptr, flags_ptr=None,
                     stream=None) -> int:
    return load_library().gq_quantize_pack(ctypes.byref(layout), w_ptr, codes_ptr, scales_ptr,
                                           zeros_ptr, flags_ptr, _stream(stream))


def gq_fake_quant(layout, w_ptr, out_dtype, out_ptr, flags_ptr=None, stream=None) -> int:
    return load_library().gq_fake_quant(ctypes.byref(layout), w_ptr, int(out_dtype), out_ptr,
                                        flags_ptr, _stream(stream))


def gq_dequant(layout, codes_ptr, scales_ptr, zeros_ptr, out_dtype, out_ptr, stream=None) -> int:
    return load_library().gq_dequant(ctypes.byref(layout), codes_ptr, scales_ptr, zeros_ptr,
                                     int(out_dtype), out_ptr, _stream(stream))


def gq_linear_workspace_bytes(layout, M: int, act: int = GQ_BF16) -> int:
    b = ctypes.c_size_t()
    st = load_library().gq_linear_workspace_bytes(ctypes.byref(layout), int(M), int(act),
                                                  ctypes.byref(b))
    if st != GQ_OK:
        raise GqError(st, "gq_linear_workspace_bytes")
    return b.value


def gq_linear(layout, M, act, x_ptr, codes_ptr, scales_ptr, zeros_ptr, y_ptr, ws_ptr, ws_bytes,
              stream=None) -> int:
    return load_library().gq_linear(ctypes.byref(layout), int(M), int(act), x_ptr, codes_ptr,
                                    scales_ptr, zeros_ptr, y_ptr, ws_ptr, int(ws_bytes),
                                    _stream(stream))


def gq_linear_noalloc(layout, M, act, x_ptr, codes_ptr, scales_ptr, zeros_ptr, y_ptr,
                      stream=None) -> int:
    return load_library().gq_linear_noalloc(ctypes.byref(layout), int(M), int(act), x_ptr,
                                            codes_ptr, scales_ptr, zeros_ptr, y_ptr,
                                            _stream(stream))


def gq_linear_dx_workspace_bytes(layout, M: int, act: int = GQ_BF16) -> int:
    b = ctypes.c_size_t()
    st = load_library().gq_linear_dx_workspace_bytes(ctypes.byref(layout), int(M), int(act),
                                                     ctypes.byref(b))
    if st != GQ_OK:
        raise GqError(st, "gq_linear_dx_workspace_bytes")
    return b.value


def gq_linear_dx(layout, M, act, dy_ptr, codes_ptr, scales_ptr, zeros_ptr, dx_ptr, ws_ptr, ws_bytes,
                 stream=None) -> int:
    return load_library().gq_linear_dx(ctypes.byref(layout), int(M), int(act), dy_ptr, codes_ptr,
                                       scales_ptr, zeros_ptr, dx_ptr, ws_ptr, int(ws_bytes),
                                       _stream(stream))


def gq_group_plan_bytes(items, M: int, act: int = GQ_BF16) -> int:
    arr = (gq_group_item * len(items))(*items)
    b = ctypes.c_size_t()
    st = load_library().gq_group_plan_bytes(len(items), arr, int(M), int(act), ctypes.byref(b))
    if st != GQ_OK:
        raise GqError(st, "gq_group_plan_bytes")
    return b.value


def gq_group_plan(items, M: int, act: int, plan_buf, plan_bytes: int) -> int:
    arr = (gq_group_item * len(items))(*items)
    return load_library().gq_group_plan(len(items), arr, int(M), int(act), plan_buf, int(plan_bytes))


def gq_linear_group(plan_buf, plan_dev_ptr, stream=None) -> int:
    return load_library().gq_linear_group(plan_buf, plan_dev_ptr, _stream(stream))


def gq_kv_attention_workspace_bytes(cache: gq_kv_cache) -> int:
    b = ctypes.c_size_t()
    st = load_library().gq_kv_attention_workspace_bytes(ctypes.byref(cache), ctypes.byref(b))
    if st != GQ_OK:
        raise GqError(st, "gq_kv_attention_workspace_bytes")
    return b.value


def gq_kv_attention(cache: gq_kv_cache, q_ptr, out_ptr, ws_ptr, ws_bytes, stream=None) -> int:
    return load_library().gq_kv_attention(ctypes.byref(cache), q_ptr, out_ptr, ws_ptr, int(ws_bytes),
                                          _stream(stream))


# ------------------------------------------------------ tensor-level API

_DT = {torch.bfloat16: GQ_BF16, torch.float16: GQ_FP16, torch.float32: GQ_FP32}


@dataclass
class Packed:
    """Packed weights of one linear: codes, fp16 scales and uint8 zeros as
    flat device tensors plus the bit map."""
    K: int
    N: int
    block_n: int
    bits: list
    codes: torch.Tensor    # uint8, 16-byte aligned
    scales: torch.Tensor   # int16 holding fp16 bit patterns
    zeros: torch.Tensor    # uint8
    flags: torch.Tensor    # int32 [1]

    @property
    def layout(self) -> gq_layout:
        lay = getattr(self, "_layout", None)
        if lay is None:
            lay = make_layout(self.K, self.N, self.block_n, self.bits)
            self._layout = lay
        return lay

    def nbytes(self) -> int:
        return self.codes.numel() + self.scales.numel() * 2 + self.zeros.numel()


def _check(st: int, where: str):
    if st != GQ_OK:
        raise GqError(st, where)


def _cuda(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_tensor(t: torch.Tensor, name: str, shape, dtype, device):
    """Refuse, before any call into the C ABI, a tensor whose shape, dtype,
    device or layout differs from what the kernels will read or write: the
    ABI sees only a pointer."""
    _cuda(t, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _check_packed(p: "Packed", device, name="packed"):
    cb, sb, zb = gq_packed_bytes(p.layout)
    if p.codes.numel() < cb or p.scales.numel() * 2 < sb or p.zeros.numel() < zb:
        raise ValueError(f"{name}: buffers smaller than its layout needs")
    for t, n in ((p.codes, "codes"), (p.scales, "scales"), (p.zeros, "zeros")):
        _cuda(t, f"{name}.{n}")
        if t.device != torch.device(device):
            raise ValueError(f"{name}.{n} must be on {device}, got {t.device}")


def empty_packed(K: int, N: int, bits, block_n: int | None = None, device="cuda") -> Packed:
    bits = [int(bits)] if isinstance(bits, int) else [int(b) for b in bits]
    block_n = N if block_n is None else int(block_n)
    lay = make_layout(K, N, block_n, bits)
    cb, sb, zb = gq_packed_bytes(lay)
    p = Packed(K, N, block_n, bits,
               torch.empty(max(cb, 16), dtype=torch.uint8, device=device),
               torch.empty(max(sb // 2, 1), dtype=torch.int16, device=device),
               torch.empty(max(zb, 1), dtype=torch.uint8, device=device),
               torch.zeros(1, dtype=torch.int32, device=device))
    p._layout = lay
    return p


def quantize_pack(w: torch.Tensor, bits, block_n: int | None = None, stream=None) -> Packed:
    """Quantize fp32 weights w [N][K] group-wise (INT4 g128 / INT2 g64).

    bits: 4, 2, 8, or a list with one entry per block of block_n output
    channels (8 marks rows kept at higher precision: groups of 128)."""
    _cuda(w, "w")
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a 2-D float32 tensor [N][K]")
    N, K = w.shape
    nb = 1 if isinstance(bits, int) else len(bits)
    if block_n is None:
        block_n = N // nb if nb else N
    block_n = max(1, int(block_n))
    p = empty_packed(K, N, bits, block_n, device=w.device)
    _check(gq_quantize_pack(p.layout, w.data_ptr(), p.codes.data_ptr(), p.scales.data_ptr(),
                            p.zeros.data_ptr(), p.flags.data_ptr(), stream), "gq_quantize_pack")
    return p


def dequant(p: Packed, dtype=torch.float32, stream=None) -> torch.Tensor:
    out = torch.empty((p.N, p.K), dtype=dtype, device=p.codes.device)
    _check(gq_dequant(p.layout, p.codes.data_ptr(), p.scales.data_ptr(), p.zeros.data_ptr(),
                      _DT[dtype], out.data_ptr(), stream), "gq_dequant")
    return out


def fake_quant(w: torch.Tensor, bits, block_n: int | None = None, dtype=torch.float32,
               flags: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Quantize-dequantize fp32 weights w [N][K] (the forward of a FakeQuantize
    module); the straight-through backward is the identity."""
    _cuda(w, "w")
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a 2-D float32 tensor [N][K]")
    N, K = w.shape
    bl = [int(bits)] if isinstance(bits, int) else [int(b) for b in bits]
    if block_n is None:
        block_n = N // len(bl) if bl else N
    lay = make_layout(K, N, max(1, int(block_n)), bl)
    out = torch.empty((N, K), dtype=dtype, device=w.device)
    fp = flags.data_ptr() if flags is not None else None
    _check(gq_fake_quant(lay, w.data_ptr(), _DT[dtype], out.data_ptr(), fp, stream), "gq_fake_quant")
    return out


_ws_cache: dict = {}
_ws_retired: list = []


def workspace(nbytes: int, device, stream=None) -> torch.Tensor | None:
    """A cached device workspace of at least nbytes, one per (device, stream):
    calls on different streams never share scratch, and calls on one stream
    are ordered by it.  A buffer that is outgrown is kept alive (never
    returned to the allocator), since a HIP graph captured earlier, or a
    kernel still queued, may hold its address."""
    if nbytes == 0:
        return None
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, _stream(stream))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _ws_retired.append(ws)
            nbytes = max(nbytes, 2 * ws.numel())
        ws = torch.empty(nbytes, dtype=torch.uint8, device=torch.device("cuda", idx))
        _ws_cache[key] = ws
    return ws


def linear(x: torch.Tensor, p: Packed, out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
           stream=None) -> torch.Tensor:
    """y = x . W_hat^T for bf16 or fp16 x [M][K]; y has x's dtype."""
    _cuda(x, "x")
    if x.dim() != 2 or x.shape[1] != p.K:
        raise ValueError(f"x must be [M][{p.K}]")
    act = _DT.get(x.dtype)
    if act not in (GQ_BF16, GQ_FP16):
        raise ValueError("x must be bfloat16 or float16")
    M = x.shape[0]
    _check_packed(p, x.device)
    y = torch.empty((M, p.N), dtype=x.dtype, device=x.device) if out is None else out
    _check_tensor(y, "out", (M, p.N), x.dtype, x.device)
    need = gq_linear_workspace_bytes(p.layout, M, act)
    if ws is None:
        ws = workspace(need, x.device, stream)
    elif ws.numel() * ws.element_size() < need or not ws.is_cuda or ws.device != x.device:
        raise ValueError(f"ws must be a device buffer on {x.device} of at least {need} bytes")
    wptr = ws.data_ptr() if ws is not None else None
    wbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(gq_linear(p.layout, M, act, x.data_ptr(), p.codes.data_ptr(), p.scales.data_ptr(),
                     p.zeros.data_ptr(), y.data_ptr(), wptr, wbytes, stream), "gq_linear")
    return y


def linear_dx(dy: torch.Tensor, p: Packed, out: torch.Tensor | None = None,
              ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """dX = dY . W_hat for bf16 or fp16 dY [M][N] (the data gradient of
    linear); dX is [M][K] in dY's dtype."""
    _cuda(dy, "dy")
    if dy.dim() != 2 or dy.shape[1] != p.N:
        raise ValueError(f"dy must be [M][{p.N}]")
    act = _DT.get(dy.dtype)
    if act not in (GQ_BF16, GQ_FP16):
        raise ValueError("dy must be bfloat16 or float16")
    M = dy.shape[0]
    _check_packed(p, dy.device)
    dx = torch.empty((M, p.K), dtype=dy.dtype, device=dy.device) if out is None else out
    _check_tensor(dx, "out", (M, p.K), dy.dtype, dy.device)
    need = gq_linear_dx_workspace_bytes(p.layout, M, act)
    if ws is None:
        ws = workspace(need, dy.device, stream)
    elif ws.numel() * ws.element_size() < need or not ws.is_cuda or ws.device != dy.device:
        raise ValueError(f"ws must be a device buffer on {dy.device} of at least {need} bytes")
    wptr = ws.data_ptr() if ws is not None else None
    wbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(gq_linear_dx(p.layout, M, act, dy.data_ptr(), p.codes.data_ptr(), p.scales.data_ptr(),
                        p.zeros.data_ptr(), dx.data_ptr(), wptr, wbytes, stream), "gq_linear_dx")
    return dx


class GroupPlan:
    """A grouped decode call: the host plan bytes, their device copy, and the
    tensors the plan points to (kept alive with it)."""

    def __init__(self, host, dev, keep, M, act):
        self.host = host
        self.dev = dev
        self._keep = keep
        self.M = M
        self.act = act


def group_plan(items, M: int | None = None) -> GroupPlan:
    """Plan y_i = x_i . W_hat_i^T for a list of (x, packed, y) triples (bf16 or
    fp16 x [M][K], M <= 4, outputs preallocated [M][N]); run it with
    linear_group(plan)."""
    if not items:
        raise ValueError("group_plan needs at least one (x, packed, y)")
    x0 = items[0][0]
    M = x0.shape[0] if M is None else int(M)
    act = _DT.get(x0.dtype)
    if act not in (GQ_BF16, GQ_FP16):
        raise ValueError("x must be bfloat16 or float16")
    dev = x0.device
    citems, keep = [], []
    for i, (x, p, y) in enumerate(items):
        _cuda(x, f"x[{i}]")
        _cuda(y, f"y[{i}]")
        if x.dtype != x0.dtype or y.dtype != x0.dtype:
            raise ValueError(f"item {i}: x and y must share the dtype of the first x")
        if tuple(x.shape) != (M, p.K) or tuple(y.shape) != (M, p.N):
            raise ValueError(f"item {i}: x must be [{M}][{p.K}] and y [{M}][{p.N}]")
        if x.device != dev or y.device != dev or p.codes.device != dev:
            raise ValueError(f"item {i}: every tensor must be on {dev}")
        citems.append(gq_group_item(p.layout, x.data_ptr(), p.codes.data_ptr(), p.scales.data_ptr(),
                                    p.zeros.data_ptr(), y.data_ptr()))
        keep.append((x, p, y))
    n = gq_group_plan_bytes(citems, M, act)
    host = ctypes.create_string_buffer(n)
    _check(gq_group_plan(citems, M, act, host, n), "gq_group_plan")
    buf = torch.frombuffer(bytearray(host.raw), dtype=torch.uint8)
    plan_dev = torch.empty(n + 16, dtype=torch.uint8, device=dev)
    off = (-plan_dev.data_ptr()) % 16
    plan_dev = plan_dev[off:off + n]
    plan_dev.copy_(buf)
    torch.cuda.synchronize(dev)
    return GroupPlan(host, plan_dev, keep, M, act)


def linear_group(plan: GroupPlan, stream=None) -> None:
    """Run every linear of a grouped plan (outputs land in the plan's y)."""
    _check(gq_linear_group(plan.host, plan.dev.data_ptr(), stream), "gq_linear_group")


def kv_cache(batch: int, q_heads: int, kv_heads: int, k: "Packed | None", v: "Packed | None",
             k_window: torch.Tensor | None = None, v_window: torch.Tensor | None = None) -> gq_kv_cache:
    """Describe a KV cache: k / v are packed caches (quantize_pack of the fp32
    cache [batch * t_packed][kv_heads * 128], one row per token) or None;
    k_window / v_window are bf16 [batch][t_window][kv_heads][128] or None."""
    if (k is None) != (v is None) or (k_window is None) != (v_window is None):
        raise ValueError("k and v (and k_window and v_window) are given together or not at all")
    if batch < 1 or kv_heads < 1:
        raise ValueError("batch and kv_heads must be positive")
    F = kv_heads * 128
    tp, bits = 0, 4
    if k is not None:
        for name, c in (("k", k), ("v", v)):
            if c.K != F or c.block_n != c.N or len(c.bits) != 1:
                raise ValueError(f"{name} must be a uniform packed cache of rows of {F} features")
            if c.N % batch != 0:
                raise ValueError(f"{name}: {c.N} rows do not split into {batch} sequences")
        if (v.N, v.bits) != (k.N, k.bits):
            raise ValueError("k and v must have the same rows and bit-width")
        tp, bits = k.N // batch, int(k.bits[0])
        _check_packed(k, k.codes.device, "k")
        _check_packed(v, k.codes.device, "v")
    tw = 0
    if k_window is not None:
        tw = k_window.shape[1] if k_window.dim() == 4 else -1
        for name, w in (("k_window", k_window), ("v_window", v_window)):
            _check_tensor(w, name, (batch, tw, kv_heads, 128), torch.bfloat16, k_window.device)
    c = gq_kv_cache(batch, q_heads, kv_heads, 128, bits, tp, tw,
                    k.codes.data_ptr() if k is not None else None,
                    k.scales.data_ptr() if k is not None else None,
                    k.zeros.data_ptr() if k is not None else None,
                    v.codes.data_ptr() if v is not None else None,
                    v.scales.data_ptr() if v is not None else None,
                    v.zeros.data_ptr() if v is not None else None,
                    k_window.data_ptr() if k_window is not None else None,
                    v_window.data_ptr() if v_window is not None else None)
    c._keep = (k, v, k_window, v_window)
    return c


def kv_attention(q: torch.Tensor, cache: gq_kv_cache, out: torch.Tensor | None = None,
                 ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One decode step of attention of bf16 q [batch][q_heads][128] over the
    cache; returns bf16 [batch][q_heads][128]."""
    _check_tensor(q, "q", (cache.batch, cache.q_heads, 128), torch.bfloat16, q.device)
    o = torch.empty_like(q) if out is None else out
    _check_tensor(o, "out", (cache.batch, cache.q_heads, 128), torch.bfloat16, q.device)
    for t in getattr(cache, "_keep", ()):
        if isinstance(t, Packed):
            _check_packed(t, q.device, "cache")
        elif isinstance(t, torch.Tensor) and t.device != q.device:
            raise ValueError(f"the cache must be on {q.device}")
    need = gq_kv_attention_workspace_bytes(cache)
    if ws is None:
        ws = workspace(need, q.device, stream)
    elif ws.numel() * ws.element_size() < need or not ws.is_cuda or ws.device != q.device:
        raise ValueError(f"ws must be a device buffer on {q.device} of at least {need} bytes")
    _check(gq_kv_attention(cache, q.data_ptr(), o.data_ptr(), ws.data_ptr(), ws.numel(), stream),
           "gq_kv_attention")
    return o
