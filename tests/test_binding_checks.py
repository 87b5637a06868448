"""The Python binding refuses mis-shaped tensors before any call into the C
ABI (the ABI sees only pointers, so a wrong-sized output or cache would be
written or read out of bounds).  CPU-only: the device test is replaced by a
stand-in that accepts host tensors, and every case raises before the ABI
call that would need a GPU."""
import pytest
import torch

gq = pytest.importorskip("quantized_gemm_groupwise_amd")


@pytest.fixture(autouse=True)
def host_tensors(monkeypatch):
    def _cuda(t, name):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    monkeypatch.setattr(gq, "_cuda", _cuda)
    monkeypatch.setattr(gq, "gq_linear", lambda *a, **k: pytest.fail("reached the ABI"))
    monkeypatch.setattr(gq, "gq_linear_dx", lambda *a, **k: pytest.fail("reached the ABI"))
    monkeypatch.setattr(gq, "gq_kv_attention", lambda *a, **k: pytest.fail("reached the ABI"))


def packed(K, N, bits=4, block_n=None, short=False):
    p = gq.empty_packed(K, N, bits, block_n, device="cpu")
    if short:
        p.codes = p.codes[:-16]
    return p


def test_linear_refuses_bad_out_ws_and_packed():
    p = packed(256, 64)
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        gq.linear(x, p, out=torch.empty((4, 63), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="bfloat16"):
        gq.linear(x, p, out=torch.empty((4, 64), dtype=torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        gq.linear(x, p, out=torch.empty((64, 4), dtype=torch.bfloat16).t())
    with pytest.raises(ValueError, match="smaller"):
        gq.linear(x, packed(256, 64, short=True))
    with pytest.raises(ValueError):
        gq.linear(torch.zeros((4, 128), dtype=torch.bfloat16), p)
    x64 = torch.zeros((64, 256), dtype=torch.bfloat16)
    need = gq.gq_linear_workspace_bytes(p.layout, 64)
    with pytest.raises(ValueError, match="ws"):
        gq.linear(x64, p, ws=torch.empty(need - 1, dtype=torch.uint8))


def test_linear_dx_refuses_bad_out():
    p = packed(256, 64)
    dy = torch.zeros((8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        gq.linear_dx(dy, p, out=torch.empty((8, 255), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="bfloat16"):
        gq.linear_dx(dy, p, out=torch.empty((8, 256), dtype=torch.float32))


def test_kv_cache_refuses_inconsistent_parts():
    B, Hkv = 2, 2
    F = Hkv * 128
    k = packed(F, B * 10)
    v = packed(F, B * 10)
    w = torch.zeros((B, 4, Hkv, 128), dtype=torch.bfloat16)
    gq.kv_cache(B, 4, Hkv, k, v, w, w.clone())                   # consistent: accepted
    with pytest.raises(ValueError, match="features"):
        gq.kv_cache(B, 4, Hkv, packed(F + 128, B * 10), v, w, w)
    with pytest.raises(ValueError, match="sequences"):
        gq.kv_cache(3, 6, Hkv, k, v, None, None)
    with pytest.raises(ValueError, match="same rows"):
        gq.kv_cache(B, 4, Hkv, k, packed(F, B * 10, bits=2), w, w)
    with pytest.raises(ValueError, match="together"):
        gq.kv_cache(B, 4, Hkv, k, None, w, w)
    with pytest.raises(ValueError, match="shape"):
        gq.kv_cache(B, 4, Hkv, k, v, w, torch.zeros((B, 5, Hkv, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="bfloat16"):
        gq.kv_cache(B, 4, Hkv, k, v, w, torch.zeros((B, 4, Hkv, 128), dtype=torch.float16))
    with pytest.raises(ValueError, match="shape"):
        gq.kv_cache(B, 4, Hkv, k, v, torch.zeros((B, 4, 128), dtype=torch.bfloat16), w)


def test_kv_attention_refuses_bad_q_and_out():
    B, Hq, Hkv = 1, 4, 2
    k = packed(Hkv * 128, 16)
    v = packed(Hkv * 128, 16)
    c = gq.kv_cache(B, Hq, Hkv, k, v)
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        gq.kv_attention(torch.zeros((B, Hq + 1, 128), dtype=torch.bfloat16), c)
    with pytest.raises(ValueError, match="shape"):
        gq.kv_attention(q, c, out=torch.empty((B, Hq, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="bfloat16"):
        gq.kv_attention(q, c, out=torch.empty((B, Hq, 128), dtype=torch.float32))


def test_layout_bits_length_is_checked():
    """The C side reads N / block_n bit-widths from the host array: a shorter
    list is refused by the binding instead of being read past its end."""
    import quantized_gemm_groupwise_amd as gq
    with pytest.raises(ValueError):
        gq.make_layout(1024, 4096, 1024, [8])
    with pytest.raises(ValueError):
        gq.make_layout(1024, 384, 128, [4, 2])
    assert gq.make_layout(1024, 256, 128, [4, 8]).N == 256
    assert gq.make_layout(1024, 0, 1, [4]).N == 0          # no block reads the entry
