"""The seeded workload recipes: shapes, budgets and block maps."""
import numpy as np

import synth as S


def test_layer_mix_budget():
    """The seeded Layer-mix assignment over the 32 x 7 Llama-3-8B linears hits
    ~2.5 bits per weight including each group's fp16 scale and uint8 zero."""
    assign = S.layer_mix_assignment()
    assert len(assign) == 224
    params = sum(N * K for (_, _, N, K, _) in assign)
    bits = sum(N * K * (b + 24 / (128 if b == 4 else 64)) for (_, _, N, K, b) in assign)
    assert 2.45 <= bits / params <= 2.5
    assert any(b == 4 for *_, b in assign) and any(b == 2 for *_, b in assign)
    assert S.layer_mix_assignment() == assign          # seeded


def test_channel_mix_block_maps():
    # 25% INT4 blocks of 128 output channels (small K keeps this cheap)
    W, bits = S.channel_mix_weight(0, N=28672, K=64)
    assert len(bits) == 224 and sum(b == 4 for b in bits) == 56
    W, bits = S.channel_mix_weight(1, N=8192, K=64)
    assert len(bits) == 64 and sum(b == 4 for b in bits) == 16


def test_outlier_channels():
    W = S.decode_weight(2, N=64, K=4096)
    colmax = np.abs(W).max(axis=0)
    assert (colmax > 0.02 * 8).sum() == round(0.005 * 4096)     # 0.5% input channels x20
    a = S.activations(4, 256, 1)
    assert a.dtype == np.uint16 and a.shape == (4, 256)
