"""Seeded synthetic inputs for group-wise INT4/INT2 weight quantization workloads.

This module is the only code shared by the CPU oracle side (tests) and the
GPU side (tests, benchmark).  It holds random draws, shapes, the bf16
rounding that turns fp32 draws into bf16 activations, and the seeded
bit-width assignments of the mixed-precision layouts.  It performs none of
the quantizer's or the matmul's arithmetic.

Every workload stands in for a real model layer that is not available here
(no checkpoints): Gaussian weights with a few outlier channels, in the
shapes of Llama-3-8B decode layers and a 70B-class MLP.  The pages describe
the outlier phenomenon (a few large values hijacking a MinMax range) in
"大模型量化实战：从原理到4-bit部署的完整指南", section 2.3 and section 4.2.
"""
from __future__ import annotations

import numpy as np

INT4, INT2 = 4, 2
GROUP = {INT4: 128, INT2: 64}

# Llama-3-8B linear shapes as (N, K): output channels N, input channels K.
LLAMA3_8B_SHAPES = {
    "up_gate": (14336, 4096),
    "down": (4096, 14336),
    "q_o": (4096, 4096),
    "k_v": (1024, 4096),
}
LLAMA3_8B_SHAPE_LIST = [LLAMA3_8B_SHAPES[k] for k in ("up_gate", "down", "q_o", "k_v")]
# The seven linears of one decoder layer, in order q, k, v, o, gate, up, down.
LLAMA3_8B_LAYER = [
    ("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
    ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336),
]
N_LAYERS = 32
# 70B-class MLP shapes for the Channel-mix prefill workload, (N, K).
MLP70B_SHAPES = [(28672, 8192), (8192, 28672)]


def bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even.

    Used only to turn fp32 Gaussian draws into bf16 activations."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def gaussian_weight(N: int, K: int, sigma: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, K), dtype=np.float32) * np.float32(sigma)


def activations(M: int, K: int, seed: int) -> np.ndarray:
    """bf16 activations ~N(0,1), returned as uint16 bit patterns [M][K]."""
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((M, K), dtype=np.float32))


# ---------------------------------------------------------------- workloads

def small_layer():
    """K=N=512 single linear, INT4 g128, weights ~N(0,0.02), M=4 bf16 rows."""
    W = gaussian_weight(512, 512, 0.02, 1001)
    x = activations(4, 512, 1002)
    return dict(W=W, x=x, block_n=512, bits=[INT4])


def decode_weight(j: int, N: int | None = None, K: int | None = None,
                  seed_base: int = 2000) -> np.ndarray:
    """Llama-3-8B-shaped weight j (0 up/gate, 1 down, 2 q/o, 3 k/v).

    ~N(0, 0.02) with 0.5% of the input channels (columns along K) scaled
    x20 to model outlier channels."""
    if N is None or K is None:
        N, K = LLAMA3_8B_SHAPE_LIST[j]
    rng = np.random.default_rng(seed_base + j)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    idx = rng.choice(K, int(round(0.005 * K)), replace=False)
    W[:, idx] *= np.float32(20.0)
    return W


def decode_x(j: int, M: int, K: int | None = None) -> np.ndarray:
    if K is None:
        K = LLAMA3_8B_SHAPE_LIST[j][1]
    return activations(M, K, 2100 + 10 * j + M)


def layer_mix_assignment(seed: int = 4999, target_bpw: float = 2.5):
    """Seeded Layer-mix bit map over the 32x7 Llama-3-8B linears.

    Linears are visited in a seeded random order; each is marked INT4 while
    the parameter-weighted average bits-per-weight (codes + fp16 scale +
    u8 zero per group) stays at or below target_bpw, the rest are INT2.
    Returns a list of (layer, name, N, K, bits) in model order."""
    linears = [(l, name, N, K) for l in range(N_LAYERS) for (name, N, K) in LLAMA3_8B_LAYER]
    bpw = {INT4: 4 + 24 / 128, INT2: 2 + 24 / 64}
    params = np.array([N * K for (_, _, N, K) in linears], dtype=np.float64)
    bits = np.full(len(linears), INT2)
    total_bits = float((params * bpw[INT2]).sum())
    total_params = float(params.sum())
    order = np.random.default_rng(seed).permutation(len(linears))
    for i in order:
        trial = total_bits + params[i] * (bpw[INT4] - bpw[INT2])
        if trial / total_params <= target_bpw:
            bits[i] = INT4
            total_bits = trial
    return [(l, name, N, K, int(b)) for (l, name, N, K), b in zip(linears, bits)]


def layer_mix_weight(layer: int, idx: int, N: int, K: int) -> np.ndarray:
    return decode_weight(0, N=N, K=K, seed_base=4000 + 7 * layer + idx)


def layer_mix_x(K: int, M: int) -> np.ndarray:
    seed = 4100 if K == 4096 else 4101
    return activations(32, K, seed)[:M]


def channel_mix_weight(j: int, N: int | None = None, K: int | None = None):
    """70B-class MLP weight j (0: N=28672,K=8192; 1: N=8192,K=28672).

    ~N(0, 0.015) with 1% of output channels scaled x30; output-channel
    blocks of 128 seeded to INT4 (25%) or INT2 (75%).  Returns (W, bits)."""
    if N is None or K is None:
        N, K = MLP70B_SHAPES[j]
    rng = np.random.default_rng(5000 + j)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.015)
    cols = rng.choice(N, int(round(0.01 * N)), replace=False)
    W[cols, :] *= np.float32(30.0)
    nblk = N // 128
    perm = rng.permutation(nblk)
    bits = np.full(nblk, INT2, dtype=np.uint8)
    bits[perm[: int(round(0.25 * nblk))]] = INT4
    return W, [int(b) for b in bits]


def channel_mix_x(j: int, M: int = 2048, K: int | None = None) -> np.ndarray:
    if K is None:
        K = MLP70B_SHAPES[j][1]
    return activations(M, K, 5100 + j)


def random_layout_bits(nblocks: int, seed: int, p_int4: float = 0.5):
    rng = np.random.default_rng(seed)
    return [INT4 if u < p_int4 else INT2 for u in rng.random(nblocks)]
