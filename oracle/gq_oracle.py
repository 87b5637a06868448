"""CPU oracle: group-wise asymmetric MinMax weight quantization, bit packing,
dequantization and the weight-only low-bit matmul.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py import this module.  The library in
quantized_gemm_groupwise_amd/ never imports it, and the two share no code
(the seeded input generators in synth/ are the only common module).

Sources (page title, then the part of the page):
  [GB]  GreenBitAI, "只需单卡 RTX 3090 低比特量化训练就能实现 LLaMA-3 8B 全参微调"
        (zeeklog) -- the two-stage quantization paragraphs: a group-wise
        MinMax quantizer, round-to-nearest, INT4 with group size 128 and
        INT2 with group size 64; Layer-mix and Channel-mix layouts.
  [LB]  "Low-bit Quantization: Slimming Large Models to the Extreme"
        (studyai.ink) -- datatype table, "Group Quantization", "Zero Point"
        (actual value = (quantized value - zero_point) x scale).
  [QP]  "大模型量化实战：从原理到4-bit部署的完整指南" (jsqmd.com) -- section 2.2:
        Q(x) = round(x/s) + z, s = (x_max - x_min)/(q_max - q_min),
        z = round(0 - x_min/s), z kept inside the integer range; section
        4.2: one layer (lm_head) kept at 8 bits inside a 4-bit model;
        section 5.1: a zero-point configuration with groups of 128.
  [GB]  also the Q-SFT and Bitorch Engine paragraphs: full-parameter
        fine-tuning in the quantized weight space, which back-propagates
        through the low-bit weights.
  [SV]  "A Survey of Low-bit Large Language Models: Basics, Systems, and
        Algorithms" (paper review) -- section 5.2 and section 6.2:
        weight-only quantization dequantizes and then runs an FP16 matmul.

Readings where the pages are silent (each one is also listed in the design
notes of the repository):
  * "round" is round-half-to-even (numpy.rint), in fp32.
  * the scale is computed in fp32, stored as fp16 rounded to nearest even,
    and the codes and the zero point are computed from the STORED fp16
    scale; a scale that rounds to zero (hi == lo, or fp16 underflow) is
    replaced by 1.0; an fp16 overflow sets FLAG_SCALE_OVERFLOW.
  * z = clamp(round(-x_min/S), 0, 2^b - 1), stored as uint8; codes are
    clamp(round(x/S) + z, 0, 2^b - 1).  A group whose zero point was clamped
    (all values of one sign, away from 0) is reported by FLAG_ZERO_CLAMPED:
    its codes saturate, and the S/2 error bound does not hold for it.
  * divisions are IEEE fp32 divisions (correctly rounded), not a reciprocal
    multiply.
  * groups run along K (the input dimension) of W stored [N][K]; codes are
    packed little-endian, 32/b codes per uint32, the lowest k in the lowest
    bits.
  * Channel-mix blocks are 128-output-channel blocks stored one after the
    other; a uniform (Layer-mix) linear is the one-block case.
  * an 8-bit block (a layer or channel block kept at higher precision) uses
    the same quantizer with q_max = 255 and groups of 128.

Parity status: every function below is pinned by tests/test_oracle_pins.py
against values the pages print, closed forms, invariants or brute force.
The bit order inside a packed word is a convention of this library (the
pages give none); it is pinned by the pack/unpack round trip and by the
dense size only.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FLAG_NONFINITE = 1
FLAG_SCALE_OVERFLOW = 2
# A finite group whose zero point round(-x_min/S) fell outside 0..2^b-1 and
# was clamped: a group that does not straddle zero (all values of one sign,
# away from 0).  Its codes saturate at the clamp, so neither "x_min -> 0,
# x_max -> 2^b-1" nor the S/2 error bound holds for it; the flag reports it.
FLAG_ZERO_CLAMPED = 4

# [GB] two-stage quantization paragraph: INT4 uses groups of 128, INT2 groups of 64.
# 8-bit rows (layers kept at higher precision inside a low-bit model, [QP]
# section 4.2: lm_head at 8 bits while the other layers stay at 4) take groups
# of 128: the pages give no 8-bit group size, and 128 is the group size of the
# zero-point weight-only configuration of [QP] section 5.1 (AWQ).
GROUP_SIZE = {4: 128, 2: 64, 8: 128}


def qmax(bits: int) -> int:
    """Largest unsigned code: 2^b - 1 ([LB] datatype table: INT4 0~15, INT2 0~3;
    8 bits give 256 values, 0..255 in the unsigned frame of [QP] section 2.2)."""
    return (1 << bits) - 1


# ------------------------------------------------------------ one quantizer

def quantize_groups(v, bits: int, clamp_zero: bool = True):
    """Asymmetric MinMax quantization of each row of v (one group per row).

    v: float32 [G][g].  Returns dict with
      codes  uint8 [G][g]   (int64 if clamp_zero is False and codes leave 0..255)
      scale  float16 [G]    the stored scale S
      s32    float32 [G]    the fp32 scale before fp16 rounding
      zero   int64 [G]      the zero point z
      lo, hi float32 [G]
      flags  int            OR of FLAG_* over all groups
      group_flags int64 [G]

    [QP] section 2.2 gives Q(x) = round(x/s) + z with
    s = (x_max - x_min) / (q_max - q_min) and z = round(0 - x_min/s);
    [GB] fixes MinMax ranges and round-to-nearest per group.
    """
    v = np.asarray(v, dtype=np.float32)
    assert v.ndim == 2
    qm = np.float32(qmax(bits))
    with np.errstate(all="ignore"):
        lo = v.min(axis=1)                         # x_min of the group
        hi = v.max(axis=1)                         # x_max of the group
        s32 = (hi - lo) / qm                       # fp32 subtract and divide, each rounded once
        s16 = s32.astype(np.float16)               # stored fp16 scale, round-half-to-even
        s16 = np.where(s16 == np.float16(0), np.float16(1.0), s16)
        S = s16.astype(np.float32)                 # exact widening
        z = np.rint(-lo / S)                       # z = round(0 - x_min / s)
        zc = (z < 0) | (z > qm)                    # outside the integer range
        if clamp_zero:
            z = np.clip(z, np.float32(0), qm)
        q = np.rint(v / S[:, None])                # round(x / s), fp32 divide
        # round(x/s) + z as an exact sum (fp64 holds both integers exactly),
        # then clamp to the code range.
        c = np.clip(q.astype(np.float64) + z.astype(np.float64)[:, None], 0.0, float(qm))
    finite = np.isfinite(v).all(axis=1)
    gflags = np.where(finite, 0, FLAG_NONFINITE)
    gflags = gflags | np.where(finite & np.isinf(s16), FLAG_SCALE_OVERFLOW, 0)
    if clamp_zero:
        gflags = gflags | np.where(finite & ~np.isinf(s16) & zc, FLAG_ZERO_CLAMPED, 0)
    c = np.where(np.isnan(c), 0.0, c)
    z64 = np.where(np.isnan(z), 0.0, z).astype(np.int64)
    codes = c.astype(np.int64)
    if clamp_zero:
        codes = codes.astype(np.uint8)
    return dict(codes=codes, scale=s16, s32=s32, zero=z64, lo=lo, hi=hi,
                flags=int(np.bitwise_or.reduce(gflags)) if gflags.size else 0,
                group_flags=gflags.astype(np.int64))


def quantize_unclamped_example(values, bits: int = 8):
    """Single group, zero point NOT clamped: the frame of the worked example
    in [QP] section 2.2 (an 8-bit range, z allowed to leave 0..255).
    Oracle-only mode used to check the formula against the page."""
    v = np.asarray(values, dtype=np.float32)[None, :]
    return quantize_groups(v, bits, clamp_zero=False)


# ------------------------------------------------------------ packing

def pack(codes, bits: int) -> np.ndarray:
    """codes uint8 [N][K] -> uint32 [N][K*b/32]; code k of a word sits at
    bits [b*(k mod 32/b), +b), lowest k lowest (little-endian)."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    per = 32 // bits
    assert K % per == 0
    c = codes.reshape(N, K // per, per).astype(np.uint32)
    shifts = (bits * np.arange(per, dtype=np.uint32))[None, None, :]
    return np.bitwise_or.reduce(c << shifts, axis=2).astype(np.uint32)


def unpack(words, bits: int, K: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint32)
    N = words.shape[0]
    per = 32 // bits
    shifts = (bits * np.arange(per, dtype=np.uint32))[None, None, :]
    c = (words[:, :, None] >> shifts) & np.uint32((1 << bits) - 1)
    return c.reshape(N, -1)[:, :K].astype(np.uint8)


# ------------------------------------------------------------ layouts

@dataclass
class Layout:
    """Bit-width map of one linear: N/block_n blocks of block_n output
    channels, each INT4 (g=128), INT2 (g=64) or INT8 (g=128, rows kept at
    higher precision).  block_n == N is a uniform (Layer-mix) linear;
    block_n == 128 is Channel-mix ([GB])."""
    K: int
    N: int
    block_n: int
    bits: list = field(default_factory=list)

    def __post_init__(self):
        assert self.N % self.block_n == 0, "N must be a multiple of block_n"
        assert len(self.bits) == self.N // self.block_n
        for b in self.bits:
            assert b in GROUP_SIZE, "bit-widths are 2, 4 or 8"
            assert self.K % GROUP_SIZE[b] == 0, "K must be a multiple of the group size"

    def blocks(self):
        """Yields (block, row0, bits, g, code_byte_offset, group_offset)."""
        cb = 0
        go = 0
        for i, b in enumerate(self.bits):
            g = GROUP_SIZE[b]
            yield i, i * self.block_n, b, g, cb, go
            cb += self.block_n * self.K * b // 8
            go += self.block_n * self.K // g

    def sizes(self):
        """(code bytes, number of scales, number of zeros)."""
        cb = sum(self.block_n * self.K * b // 8 for b in self.bits)
        ng = sum(self.block_n * self.K // GROUP_SIZE[b] for b in self.bits)
        return cb, ng, ng


@dataclass
class Packed:
    layout: Layout
    codes: np.ndarray      # uint8, all blocks back to back
    scales: np.ndarray     # uint16 fp16 bit patterns
    zeros: np.ndarray      # uint8
    flags: int


def quantize_pack(W, layout: Layout) -> Packed:
    """Quantize W fp32 [N][K] block by block and pack the codes."""
    W = np.asarray(W, dtype=np.float32)
    assert W.shape == (layout.N, layout.K)
    cb, ng, _ = layout.sizes()
    codes = np.zeros(cb, dtype=np.uint8)
    scales = np.zeros(ng, dtype=np.uint16)
    zeros = np.zeros(ng, dtype=np.uint8)
    flags = 0
    K = layout.K
    for _, r0, b, g, coff, goff in layout.blocks():
        rows = W[r0:r0 + layout.block_n]
        q = quantize_groups(rows.reshape(-1, g), b)
        words = pack(q["codes"].reshape(layout.block_n, K), b)
        nbytes = layout.block_n * K * b // 8
        codes[coff:coff + nbytes] = words.astype("<u4").view(np.uint8).reshape(-1)
        n = layout.block_n * K // g
        scales[goff:goff + n] = q["scale"].view(np.uint16)
        zeros[goff:goff + n] = q["zero"].astype(np.uint8)
        flags |= q["flags"]
    return Packed(layout, codes, scales, zeros, flags)


def block_fields(p: Packed, block: int):
    """Codes uint8 [block_n][K], scale fp16 [block_n][K/g], zero [block_n][K/g]."""
    L = p.layout
    for i, r0, b, g, coff, goff in L.blocks():
        if i == block:
            nbytes = L.block_n * L.K * b // 8
            words = p.codes[coff:coff + nbytes].view("<u4").reshape(L.block_n, -1)
            c = unpack(words, b, L.K)
            n = L.block_n * L.K // g
            s = p.scales[goff:goff + n].view(np.float16).reshape(L.block_n, -1)
            z = p.zeros[goff:goff + n].reshape(L.block_n, -1)
            return c, s, z, b, g
    raise IndexError(block)


def dequant(p: Packed, rows=None) -> np.ndarray:
    """W_hat[n,k] = (c - z) * S in fp32 ([LB] "Zero Point").

    The product is exact in fp32: |c - z| <= 255 has at most 8 bits and S
    has an 11-bit significand.  rows: optional iterable of output channels."""
    L = p.layout
    sel = np.arange(L.N) if rows is None else np.asarray(list(rows), dtype=np.int64)
    out = np.zeros((len(sel), L.K), dtype=np.float32)
    blk_of = sel // L.block_n
    for blk in np.unique(blk_of):
        c, s, z, b, g = block_fields(p, int(blk))
        pos = np.nonzero(blk_of == blk)[0]
        r = sel[pos] - int(blk) * L.block_n
        S = np.repeat(s[r].astype(np.float64), g, axis=1)
        Z = np.repeat(z[r].astype(np.float64), g, axis=1)
        with np.errstate(invalid="ignore"):
            w64 = (c[r].astype(np.float64) - Z) * S
            w32 = w64.astype(np.float32)
            assert np.array_equal(w32.astype(np.float64), w64, equal_nan=True), \
                "dequantized value not exact in fp32"
        out[pos] = w32
    return out


def dequant_as(p: Packed, dtype: str) -> np.ndarray:
    """Dequantized weights rounded to the requested storage type:
    'fp32' (exact), 'fp16' (round-half-to-even) or 'bf16' (uint16 bits, RNE)."""
    w = dequant(p)
    if dtype == "fp32":
        return w
    if dtype == "fp16":
        with np.errstate(over="ignore"):
            return w.astype(np.float16)
    if dtype == "bf16":
        return f64_to_bf16_bits(w.astype(np.float64))
    raise ValueError(dtype)


def fake_quant(W, layout: Layout, dtype: str = "fp32") -> np.ndarray:
    """Quantize, then dequantize, without packing ([QP] section 5.2: a
    FakeQuantize module simulates round(x/s) + z in the forward pass; the
    backward lets the gradient through the FP32 path, i.e. the identity).

    The quantizer is the group-wise MinMax one of quantize_pack and the
    dequantizer the one of dequant, applied in that order; dtype as for
    dequant_as ('fp32' exact, 'fp16', 'bf16' bits)."""
    return dequant_as(quantize_pack(W, layout), dtype)


# ------------------------------------------------------------ matmul

def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def linear(x_bf16, p: Packed, rows=None) -> np.ndarray:
    """y = x . W_hat^T accumulated in fp64 ([SV] section 5.2: weight-only
    quantization dequantizes, then runs the matmul in floating point).

    x_bf16: uint16 bf16 bit patterns [M][K] (exactly representable in fp64).
    rows: optional subset of output channels; returns fp64 [M][len(rows)]."""
    x = bf16_bits_to_f64(x_bf16)
    w = dequant(p, rows).astype(np.float64)
    return x @ w.T


def linear_dx(dy_bf16, p: Packed, cols=None) -> np.ndarray:
    """dX = dY . W_hat accumulated in fp64: the data gradient of
    y = x . W_hat^T, which back-propagation through the quantized linear
    needs when the model is fine-tuned in its quantized space ([GB] Q-SFT
    and Bitorch Engine paragraphs: gradients through low-bit weights).
    W_hat is the dequantized weight of dequant ([LB] "Zero Point").

    dy_bf16: uint16 bf16 bit patterns [M][N].  cols: optional subset of input
    channels k; returns fp64 [M][len(cols)] (all K when cols is None)."""
    dy = bf16_bits_to_f64(dy_bf16)
    w = dequant(p).astype(np.float64)
    if cols is not None:
        w = w[:, np.asarray(list(cols), dtype=np.int64)]
    return dy @ w


# ------------------------------------------------- KV-cache attention

def kv_cache_pack(kv, bits: int) -> Packed:
    """Quantize a key or value cache for the decode attention: kv is fp32
    [tokens][kv_heads * head_dim]; each token row is quantized group-wise
    along its features exactly as a weight row ([SV] KV-cache bullet: the
    cache is compressed with the same INT4 / INT2 formats), i.e. one
    uniform layout whose "output channels" are tokens."""
    kv = np.asarray(kv, dtype=np.float32)
    return quantize_pack(kv, Layout(kv.shape[1], kv.shape[0], max(1, kv.shape[0]), [bits]))


def kv_decode_attention(q_bf16, k_packed, v_packed, k_window_bf16, v_window_bf16,
                        batch: int, q_heads: int, kv_heads: int, head_dim: int,
                        return_abs: bool = False):
    """One decode step of attention over a group-wise quantized KV cache, in
    fp64 ([SV] KV-cache bullet and its techniques: the cache is stored at low
    bit width and dequantized for attention; the newest tokens stay in full
    precision in a window and are not quantized).

    q_bf16: uint16 bf16 bits [batch][q_heads][head_dim].
    k_packed / v_packed: Packed caches of batch * t_packed token rows (the
      rows of sequence b are rows b * t_packed ..), or None when t_packed = 0.
    k_window_bf16 / v_window_bf16: uint16 bf16 bits
      [batch][t_window][kv_heads][head_dim] (t_window may be 0).
    Query head h attends with key/value head h // (q_heads // kv_heads);
    scores are q . k / sqrt(head_dim) over the packed tokens followed by the
    window tokens; softmax; the output is the probability-weighted sum of the
    values.  Returns fp64 [batch][q_heads][head_dim]; with return_abs, also
    sum_t p_t |v_t| per output (the scale an error bound of P . V takes)."""
    G = q_heads // kv_heads
    q = bf16_bits_to_f64(q_bf16).reshape(batch, q_heads, head_dim)
    kw = bf16_bits_to_f64(k_window_bf16).reshape(batch, -1, kv_heads, head_dim)
    vw = bf16_bits_to_f64(v_window_bf16).reshape(batch, -1, kv_heads, head_dim)
    if k_packed is not None:
        tp = k_packed.layout.N // batch
        kp = dequant(k_packed).astype(np.float64).reshape(batch, tp, kv_heads, head_dim)
        vp = dequant(v_packed).astype(np.float64).reshape(batch, tp, kv_heads, head_dim)
        keys = np.concatenate([kp, kw], axis=1)
        vals = np.concatenate([vp, vw], axis=1)
    else:
        keys, vals = kw, vw
    out = np.zeros((batch, q_heads, head_dim))
    absw = np.zeros((batch, q_heads, head_dim))
    for b in range(batch):
        for h in range(q_heads):
            kh = h // G
            s = keys[b, :, kh, :] @ q[b, h] / np.sqrt(head_dim)
            e = np.exp(s - s.max())
            p = e / e.sum()
            out[b, h] = p @ vals[b, :, kh, :]
            absw[b, h] = p @ np.abs(vals[b, :, kh, :])
    return (out, absw) if return_abs else out


def f64_to_bf16_bits(a) -> np.ndarray:
    """Round fp64 values to bf16 (8 significant bits), nearest-even, with
    bf16 subnormals and overflow to infinity; returns uint16 bit patterns."""
    a = np.asarray(a, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.float64)
    with np.errstate(all="ignore"):
        m, e = np.frexp(a)                       # a = m * 2^e, 0.5 <= |m| < 1
        e = np.maximum(e, -125)                  # bf16 min normal exponent: 2^-126 = 0.5*2^-125
        scaled = np.ldexp(a, 8 - e)              # significand in units of the last bf16 bit
        r = np.ldexp(np.rint(scaled), e - 8)
        out[...] = r
        big = np.abs(r) > 3.3895313892515355e38  # beyond the largest finite bf16
        out[big] = np.copysign(np.inf, a[big])
    out[np.isnan(a)] = np.nan
    f = out.astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    bits[np.isnan(a)] = 0x7FC0
    return bits


def compare_linear(y_gpu_bf16, y_ref):
    """Acceptance numbers for a linear result.

    normwise: ||y_gpu - y_ref||_F / ||y_ref||_F against the fp64 oracle.
    match:    fraction of elements equal to the oracle rounded to bf16.
    max_ulp:  largest difference in bf16 units of the last place."""
    yg = bf16_bits_to_f64(y_gpu_bf16)
    denom = np.linalg.norm(y_ref)
    normwise = float(np.linalg.norm(yg - y_ref) / denom) if denom > 0 else float(np.linalg.norm(yg))
    rb = f64_to_bf16_bits(y_ref)
    match = float(np.mean(rb == np.asarray(y_gpu_bf16, dtype=np.uint16)))
    ordered = lambda b: np.where(b & 0x8000, -(b.astype(np.int64) & 0x7FFF), b.astype(np.int64))
    ulp = int(np.max(np.abs(ordered(rb) - ordered(np.asarray(y_gpu_bf16, dtype=np.uint16))))) if rb.size else 0
    return dict(normwise=normwise, match=match, max_ulp=ulp)
