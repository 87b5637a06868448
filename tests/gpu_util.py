"""Helpers for the GPU parity tests: move seeded numpy inputs to the device,
call the library through its C-ABI binding, bring results back."""
import numpy as np
import torch

import quantized_gemm_groupwise_amd as gq


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(bits.view(np.int16), None).view(torch.bfloat16)


def gpu_quantize(W: np.ndarray, block_n: int, bits):
    """Quantize on the GPU; returns (codes u8, scales u16, zeros u8, flags, Packed)."""
    p = gq.quantize_pack(to_dev(W), bits, block_n)
    torch.cuda.synchronize()
    cb, sb, zb = gq.gq_packed_bytes(p.layout)
    codes = p.codes.cpu().numpy()[:cb]
    scales = p.scales.cpu().numpy().view(np.uint16)[: sb // 2]
    zeros = p.zeros.cpu().numpy()[:zb]
    return codes, scales, zeros, int(p.flags.cpu().item()), p


def upload_packed(op, device="cuda") -> "gq.Packed":
    """An oracle Packed as a library Packed (device buffers)."""
    L = op.layout
    p = gq.empty_packed(L.K, L.N, L.bits, L.block_n, device=device)
    p.codes[: op.codes.size].copy_(torch.from_numpy(op.codes))
    p.scales[: op.scales.size].copy_(torch.from_numpy(op.scales.view(np.int16)))
    p.zeros[: op.zeros.size].copy_(torch.from_numpy(op.zeros))
    return p


def y_bits(y: torch.Tensor) -> np.ndarray:
    return y.view(torch.int16).cpu().numpy().view(np.uint16)
