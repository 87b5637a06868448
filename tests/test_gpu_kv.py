"""GPU parity of the decode attention over a group-wise quantized KV cache
(gq_kv_attention) against the fp64 oracle (oracle.kv_decode_attention) on
the same seeded inputs; the packed caches come from the oracle's packing
(byte-identical to gq_quantize_pack) uploaded to the device.

Bar: normwise relative error <= 2e-3 over the output against the fp64
oracle, and elementwise |out - ref| <= 2^-8 |ref| + 2^-12 sum_t p_t |v_t|
(bf16 output rounding, plus the fp32 arithmetic of the scores -- computed
from exact fp16 forms with fp32 accumulation --, the softmax and P . V,
whose errors scale with the probability-weighted magnitude of the values,
not with the largest value of the cache).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

gq = pytest.importorskip("quantized_gemm_groupwise_amd")
from tests.gpu_util import bf16_dev, upload_packed, y_bits  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load_library()


def _say(*a):
    print(*a, flush=True)


def kv_inputs(seed, B, Hq, Hkv, tp, tw, bits, kscale=1.0):
    """Synthetic decode-step inputs: q and keys Gaussian (keys times kscale,
    which sets how peaked the softmax is), values Gaussian; fp32 caches
    quantized by the oracle, the window rounded to bf16."""
    rng = np.random.default_rng(seed)
    D = 128
    q = S.bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32))
    k = (rng.standard_normal((B * tp, Hkv * D)) * kscale).astype(np.float32)
    v = rng.standard_normal((B * tp, Hkv * D)).astype(np.float32)
    kp = O.kv_cache_pack(k, bits) if tp else None
    vp = O.kv_cache_pack(v, bits) if tp else None
    kw = S.bf16_bits((rng.standard_normal((B, tw, Hkv, D)) * kscale).astype(np.float32))
    vw = S.bf16_bits(rng.standard_normal((B, tw, Hkv, D)).astype(np.float32))
    return q, kp, vp, kw, vw


def run_gpu(q, kp, vp, kw, vw, B, Hq, Hkv):
    kd = upload_packed(kp) if kp is not None else None
    vd = upload_packed(vp) if vp is not None else None
    tw = kw.shape[1]
    kwd = bf16_dev(np.ascontiguousarray(kw)) if tw else None
    vwd = bf16_dev(np.ascontiguousarray(vw)) if tw else None
    cache = gq.kv_cache(B, Hq, Hkv, kd, vd, kwd, vwd)
    out = gq.kv_attention(bf16_dev(q), cache)
    torch.cuda.synchronize()
    return y_bits(out).reshape(B, Hq, 128)


def oracle(q, kp, vp, kw, vw, B, Hq, Hkv):
    """(fp64 output, sum_t p_t |v_t| per output)."""
    return O.kv_decode_attention(q, kp, vp, kw, vw, B, Hq, Hkv, 128, return_abs=True)


def gate(out_bits, ref_abs):
    """Normwise over the whole output, plus the elementwise bound; returns
    (normwise, normwise of the bf16 rounding of the exact result alone,
    largest error beyond the bf16 rounding term in units of sum p|v|)."""
    ref, absw = ref_abs
    got = O.bf16_bits_to_f64(out_bits)
    normwise = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    rounding = np.linalg.norm(O.bf16_bits_to_f64(O.f64_to_bf16_bits(ref)) - ref) / np.linalg.norm(ref)
    assert normwise <= 2e-3, (normwise, rounding)
    over = np.maximum(np.abs(got - ref) - 2.0 ** -8 * np.abs(ref), 0)
    excess = np.max(np.where(absw > 0, over / np.where(absw > 0, absw, 1), np.where(over > 0, np.inf, 0)))
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -12 * absw
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{bad.sum()} elements outside the bound (excess {excess:.3e} of sum p|v|)"
    return normwise, rounding, excess


@pytest.mark.parametrize("B,Hq,Hkv,tp,tw,bits", [
    (1, 32, 8, 256, 16, 4),        # Llama-3-8B heads, whole tiles, window
    (1, 32, 8, 100, 0, 4),         # ragged last tile, no window
    (2, 32, 8, 77, 5, 2),          # INT2, two sequences, ragged
    (1, 8, 8, 33, 1, 4),           # one query head per key/value head
    (3, 16, 2, 129, 7, 2),         # 8 query heads per key/value head, 3 sequences
    (1, 4, 4, 1, 0, 4),            # a single packed token
    (1, 32, 8, 0, 40, 4),          # window only
    (1, 12, 6, 300, 9, 4),         # two workgroup head groups, the second with 2 heads
    (1, 2, 1, 500, 3, 2),          # one key/value head
    (2, 8, 2, 40, 100, 2),         # more window parts than packed splits
    (16, 32, 8, 70, 5, 4),         # 512 (sequence, head) pairs: combine over all features per workgroup
    (1, 6, 3, 100, 4, 4),          # 3 key/value heads: a group of 3 in a 4-head tile
    (2, 14, 7, 90, 3, 2),          # 7 key/value heads, INT2: groups of 4 and 3
])
def test_kv_attention_shapes(B, Hq, Hkv, tp, tw, bits):
    q, kp, vp, kw, vw = kv_inputs(100 + tp + tw, B, Hq, Hkv, tp, tw, bits)
    _say("kv", B, Hq, Hkv, tp, tw, bits)
    got = run_gpu(q, kp, vp, kw, vw, B, Hq, Hkv)
    _say("normwise", gate(got, oracle(q, kp, vp, kw, vw, B, Hq, Hkv)))


@pytest.mark.parametrize("kscale", [0.05, 3.0])
def test_kv_attention_flat_and_peaked(kscale):
    """Nearly uniform and strongly peaked softmax (scores up to ~100)."""
    B, Hq, Hkv, tp, tw = 1, 32, 8, 1000, 24
    q, kp, vp, kw, vw = kv_inputs(7, B, Hq, Hkv, tp, tw, 4, kscale=kscale)
    got = run_gpu(q, kp, vp, kw, vw, B, Hq, Hkv)
    _say("normwise", gate(got, oracle(q, kp, vp, kw, vw, B, Hq, Hkv)))


def test_kv_attention_long_context():
    """32768 tokens (32640 packed + 128 window), Llama-3-8B heads, INT4:
    the configuration the benchmark times, with its split over 255 parts."""
    B, Hq, Hkv, tp, tw = 1, 32, 8, 32640, 128
    q, kp, vp, kw, vw = kv_inputs(8, B, Hq, Hkv, tp, tw, 4)
    _say("kv long context", tp, tw)
    got = run_gpu(q, kp, vp, kw, vw, B, Hq, Hkv)
    _say("normwise", gate(got, oracle(q, kp, vp, kw, vw, B, Hq, Hkv)))


def test_kv_attention_gpu_packing_and_repeat():
    """The cache packed on the GPU by gq_quantize_pack (one row per token)
    gives the oracle's answer; a second call gives the same bytes."""
    B, Hq, Hkv, tp, tw = 2, 32, 8, 200, 8
    rng = np.random.default_rng(9)
    q = S.bf16_bits(rng.standard_normal((B, Hq, 128)).astype(np.float32))
    k = rng.standard_normal((B * tp, Hkv * 128)).astype(np.float32)
    v = rng.standard_normal((B * tp, Hkv * 128)).astype(np.float32)
    kw = S.bf16_bits(rng.standard_normal((B, tw, Hkv, 128)).astype(np.float32))
    vw = S.bf16_bits(rng.standard_normal((B, tw, Hkv, 128)).astype(np.float32))
    kd = gq.quantize_pack(torch.from_numpy(k).cuda(), 2)
    vd = gq.quantize_pack(torch.from_numpy(v).cuda(), 2)
    cache = gq.kv_cache(B, Hq, Hkv, kd, vd, bf16_dev(kw), bf16_dev(vw))
    qd = bf16_dev(q)
    a = y_bits(gq.kv_attention(qd, cache))
    b2 = y_bits(gq.kv_attention(qd, cache))
    torch.cuda.synchronize()
    assert np.array_equal(a, b2)
    kp, vp = O.kv_cache_pack(k, 2), O.kv_cache_pack(v, 2)
    gate(a.reshape(B, Hq, 128), oracle(q, kp, vp, kw, vw, B, Hq, Hkv))


@pytest.mark.parametrize("qexp", [60, -60, None])
def test_kv_attention_query_rescale_range(qexp):
    """Query rows far from 1 in magnitude (2^60, 2^-60) and a query spanning
    2^40 within each head (largest components near 1): the per-head power-of-two rescale that makes q
    exact in fp16 must keep the scores right (a huge query gives a one-hot
    softmax, a tiny one a uniform softmax)."""
    B, Hq, Hkv, tp, tw = 1, 8, 2, 300, 6
    q, kp, vp, kw, vw = kv_inputs(11, B, Hq, Hkv, tp, tw, 4, kscale=0.3)
    qf = S.bf16_to_f32(q).astype(np.float64)
    if qexp is None:
        # largest components near 1, so the scores stay well conditioned
        span = 2.0 ** np.linspace(-40, 0, 128)
        qf = qf * span[None, None, np.random.default_rng(12).permutation(128)]
    else:
        qf = qf * 2.0 ** qexp
    q = S.bf16_bits(qf.astype(np.float32))
    got = run_gpu(q, kp, vp, kw, vw, B, Hq, Hkv)
    _say("q rescale", qexp, gate(got, oracle(q, kp, vp, kw, vw, B, Hq, Hkv)))


def test_kv_attention_errors():
    c = gq.gq_kv_cache(1, 32, 8, 64, 4, 10, 0, None, None, None, None, None, None, None, None)
    with pytest.raises(gq.GqError) as e:
        gq.gq_kv_attention_workspace_bytes(c)
    assert e.value.status == gq.GQ_ERR_SHAPE
    c = gq.gq_kv_cache(1, 12, 8, 128, 4, 10, 0, None, None, None, None, None, None, None, None)
    with pytest.raises(gq.GqError):
        gq.gq_kv_attention_workspace_bytes(c)
    c = gq.gq_kv_cache(1, 32, 8, 128, 3, 10, 0, None, None, None, None, None, None, None, None)
    with pytest.raises(gq.GqError) as e:
        gq.gq_kv_attention_workspace_bytes(c)
    assert e.value.status == gq.GQ_ERR_BITS
    c = gq.gq_kv_cache(1, 32, 8, 128, 4, 0, 0, None, None, None, None, None, None, None, None)
    with pytest.raises(gq.GqError):
        gq.gq_kv_attention_workspace_bytes(c)
