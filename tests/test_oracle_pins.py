"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, never against the oracle's own formulas.

Each test names the passage it follows.  A plausible slip in the oracle
(a dropped zero point, round((x-lo)/s) instead of round(x/s)+z, a wrong
q_max, a transposed operand, truncating instead of rounding the scale)
fails at least one of them; test_planted_mistakes_are_caught plants such
slips in a copy of the oracle on the CPU and checks that they are caught.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth as S


def rne(fr: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even (exact)."""
    return round(fr)


# ----------------------------------------------------------------- P1 levels

@pytest.mark.parametrize("bits", [4, 2, 8])
def test_levels_on_decode_like_weights(bits, golden):
    """INT4 has 16 levels, INT2 has 4 and INT8 256 (datatype table and the
    count of INT4 values in Low-bit Quantization: Slimming Large Models to the
    Extreme; the 0..255 frame of section 2.2 of '大模型量化实战'); all of them
    occur on Gaussian weights with outlier channels.  The 8-bit group size is
    the zero-point configuration's 128 (section 5.1 of the same page)."""
    key = {4: "INT4", 2: "INT2", 8: "INT8"}[bits]
    lv = golden["levels"][key]
    assert O.qmax(bits) == lv["unsigned_max"] and lv["levels"] == O.qmax(bits) + 1
    if bits == 8:
        assert O.GROUP_SIZE[bits] == golden["awq_group_size"]["value"]
    else:
        assert O.GROUP_SIZE[bits] == golden["group_sizes"][key]
    W = S.decode_weight(3, N=128, K=4096)
    g = O.GROUP_SIZE[bits]
    q = O.quantize_groups(W.reshape(-1, g), bits)
    codes = q["codes"]
    assert codes.min() >= lv["unsigned_min"] and codes.max() <= lv["unsigned_max"]
    assert len(np.unique(codes)) == lv["levels"]
    assert q["flags"] == 0


# --------------------------------------------------- P2 exact-scale groups

def _exact_group(bits, S0, ka, us, R=256):
    """Group whose scale is exactly S0: v = (u/R - ka/R) * S0."""
    Q = O.qmax(bits)
    us = sorted(set([0, R * Q] + list(us)))
    v = np.array([(u - ka) / R * S0 for u in us], dtype=np.float64)
    v32 = v.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), v)      # exact in fp32 by construction
    return us, v32


@pytest.mark.parametrize("bits", [4, 2, 8])
def test_exact_scale_groups(bits):
    """x_min -> 0, x_max -> 2^b - 1, |W_hat - W| <= S/2, ties to even.

    With lo = -a*S0 and hi = (q_max - a)*S0 every step is exact, so the
    affine map of section 2.2 of '大模型量化实战' (s = range/(q_max-q_min),
    z = round(-x_min/s), Q = round(x/s) + z) has a closed-form result that
    is computed here in exact rational arithmetic."""
    rng = np.random.default_rng(7)
    Q = O.qmax(bits)
    g = O.GROUP_SIZE[bits]
    # sub-step resolution: values are multiples of S0/R; 8-bit groups span
    # 255 steps, so a coarser R keeps every value exact in fp32
    R = 256 if bits <= 4 else 8
    for trial in range(60):
        e = int(rng.integers(-14, 3))
        S0 = float(np.float16(2.0 ** e * (1 + int(rng.integers(0, 1024)) / 1024)))
        while True:
            ka = int(rng.integers(1, R * Q))
            if ka % R != R // 2:
                break
        # ties: t - a = n + 1/2 for a few n
        ties = [ka + R // 2 + R * n for n in range(-Q, Q) if 0 <= ka + R // 2 + R * n <= R * Q][:4]
        us = list(rng.integers(0, R * Q + 1, size=g - 2 - len(ties))) + ties
        us, v = _exact_group(bits, S0, ka, us, R)
        v = np.concatenate([v, np.full(g - len(v), v[0], np.float32)]) if len(v) < g else v[:g]
        q = O.quantize_groups(v[None, :], bits)
        S = float(q["scale"][0])
        assert S == S0
        z = int(q["zero"][0])
        assert z == rne(Fraction(ka, R))
        c = q["codes"][0].astype(int)
        expect = [min(max(rne(Fraction(int(u) - ka, R)) + z, 0), Q) for u in
                  (list(us) + [us[0]] * (g - len(us)))[:g]]
        assert list(c) == expect
        lo_i, hi_i = int(np.argmin(v)), int(np.argmax(v))
        assert c[lo_i] == 0 and c[hi_i] == Q
        w_hat = (c - z) * S
        assert np.all(np.abs(w_hat - v.astype(np.float64)) <= S / 2)
        for u in ties:
            i = list(us).index(u)
            n2 = (u - ka) // (R // 2)                  # t - a = n2 / 2, n2 odd
            assert (c[i] - z) % 2 == 0 and abs(2 * (c[i] - z) - n2) == 1


# ------------------------------------------------- one-sided groups

@pytest.mark.parametrize("bits", [4, 2, 8])
def test_zero_clamp_flag_one_sided_groups(bits):
    """A group that does not straddle zero has round(-x_min/S) outside the
    code range ([QP] 2.2 keeps z inside it), so z is clamped and the codes
    saturate; such a group, and only such a group, carries FLAG_ZERO_CLAMPED.
    Constructed with an exactly representable scale S = 2^-4: the values
    below are multiples of S/8, so every quotient v/S is exact."""
    Q = O.qmax(bits)
    g = O.GROUP_SIZE[bits]
    S0 = 2.0 ** -4
    def grp(lo_steps, hi_steps):
        v = np.full(g, lo_steps * S0, np.float32)
        v[1] = hi_steps * S0
        v[2:] = np.linspace(lo_steps, hi_steps, g - 2).round(3).astype(np.float32) * np.float32(S0)
        v[2:] = np.clip(np.round(v[2:] / (S0 / 8)) * (S0 / 8), lo_steps * S0, hi_steps * S0)
        return v
    rows = [grp(5, 5 + Q),        # all positive: -lo/S = -5 -> z clamps to 0
            grp(-5 - Q, -5),      # all negative: -lo/S = 5 + Q -> z clamps to Q
            grp(-2, Q - 2),       # straddles zero: z = 2, no flag
            grp(0, Q)]            # touches zero: z = 0 exactly, no flag
    q = O.quantize_groups(np.stack(rows), bits)
    assert np.all(q["scale"].astype(np.float64) == S0)
    assert list(q["group_flags"]) == [O.FLAG_ZERO_CLAMPED, O.FLAG_ZERO_CLAMPED, 0, 0]
    assert q["flags"] == O.FLAG_ZERO_CLAMPED
    assert list(q["zero"]) == [0, Q, 2, 0]
    c = q["codes"].astype(np.int64)
    # positive group: codes are round(v/S) clamped at Q, so the largest values saturate
    assert c[0, 0] == min(5, Q) and c[0, 1] == Q
    # negative group: codes round(v/S) + Q clamped at 0
    assert c[1, 0] == 0 and c[1, 1] == max(Q - 5, 0)
    # the straddling groups keep the endpoint and S/2 statements
    for r in (2, 3):
        assert c[r, 0] == 0 and c[r, 1] == Q
        err = np.abs((c[r] - q["zero"][r]) * S0 - rows[r].astype(np.float64))
        assert np.all(err <= S0 / 2)


# ------------------------------------------------- P3 random-data endpoints

@pytest.mark.parametrize("bits", [4, 2, 8])
def test_endpoint_and_error_bounds_random(bits):
    """Endpoint and error statements that survive the fp16 scale rounding.

    c(x_min) = 0 where z was not clamped; c(x_max) is q_max or q_max-1, the
    latter only when the stored scale rounded up; every element is within
    S/2 + max(0, range - q_max*S) + 2^-16*S of its dequantized value."""
    Q = O.qmax(bits)
    g = O.GROUP_SIZE[bits]
    W = S.decode_weight(2, N=256, K=4096)
    G = W.reshape(-1, g)
    q = O.quantize_groups(G, bits)
    Sv = q["scale"].astype(np.float64)
    z = q["zero"]
    c = q["codes"].astype(np.int64)
    lo, hi = q["lo"].astype(np.float64), q["hi"].astype(np.float64)
    raw_z = np.rint(-q["lo"] / q["scale"].astype(np.float32))
    assert np.all(raw_z == z)                          # no clamped zero on this data
    assert q["flags"] == 0                             # and none reported
    rows = np.arange(G.shape[0])
    c_lo = c[rows, np.argmin(G, axis=1)]
    c_hi = c[rows, np.argmax(G, axis=1)]
    assert np.all(c_lo == 0)
    assert np.all((c_hi == Q) | (c_hi == Q - 1))
    s32 = q["s32"].astype(np.float64)
    assert np.all(Sv[c_hi == Q - 1] >= s32[c_hi == Q - 1])
    err = np.abs((c - z[:, None]) * Sv[:, None] - G.astype(np.float64))
    bound = Sv / 2 + np.maximum(0.0, (hi - lo) - Q * Sv) + Sv * 2.0 ** -16
    assert np.all(err <= bound[:, None])
    # and almost everywhere the plain S/2 bound
    assert np.mean(err <= Sv[:, None] / 2) > 0.999


# ----------------------------------------------------- fake quantization

def test_fake_quant_hand_example():
    """One INT2 group of the 64 weights k/16 (k = 0..63) through FakeQuantize
    ("大模型量化实战", section 5.2: round(x/s) + z in the forward, then back).
    x_min = 0 and x_max = 63/16 give s = (63/16)/3 = 21/16, exact in fp16, and
    z = round(0) = 0, so the code is round(k/21): 0 up to k = 10, 1 from 11
    to 31, 2 from 32 to 52 and 3 from 53 on; the output is code * 21/16."""
    w = (np.arange(64, dtype=np.float32) / 16).reshape(1, 64)
    out = O.fake_quant(w, O.Layout(64, 1, 1, [2]))
    code = np.array([0] * 11 + [1] * 21 + [2] * 21 + [3] * 11)
    assert np.array_equal(out[0].astype(np.float64), code * 21 / 16)


@pytest.mark.parametrize("bits", [4, 2, 8])
def test_fake_quant_keeps_values_on_the_grid(bits):
    """A group whose values already sit on a 2^b-level grid spanning it
    (v = j/2^b - 1/2 with j = 0 and j = 2^b - 1 present) comes back unchanged:
    s = (2^b - 1)/2^b / (2^b - 1) = 2^-b, z = 2^(b-1), code = j."""
    g = O.GROUP_SIZE[bits]
    lv = 2 ** bits
    j = np.concatenate([[0, lv - 1], np.arange(g - 2) % lv])
    w = (j / lv - 0.5).astype(np.float32).reshape(1, g)
    out = O.fake_quant(w, O.Layout(g, 1, 1, [bits]))
    assert np.array_equal(out, w)


@pytest.mark.parametrize("bits", [4, 2, 8])
def test_fake_quant_levels_and_error(bits):
    """Each output group takes at most 2^b values (16 for INT4, 4 for INT2,
    256 for INT8: datatype table of "Low-bit Quantization"), evenly spaced, and stays within
    half a step of the input wherever the zero point was not clamped, plus the
    part of the range past (2^b - 1) steps when the fp16 scale rounded down."""
    g = O.GROUP_SIZE[bits]
    W = S.decode_weight(1, N=64, K=1024)
    fq = O.fake_quant(W, O.Layout(1024, 64, 64, [bits])).astype(np.float64).reshape(-1, g)
    G = W.astype(np.float64).reshape(-1, g)
    for out, w in zip(fq, G):
        vals = np.unique(out)
        assert len(vals) <= 2 ** bits
        step = np.min(np.diff(vals))
        assert np.allclose((vals - vals[0]) / step, np.rint((vals - vals[0]) / step), atol=1e-9)
        if w.min() < 0 < w.max():
            over = max(0.0, (w.max() - w.min()) - O.qmax(bits) * step)
            assert np.max(np.abs(out - w)) <= (step / 2 + over) * (1 + 2 ** -10)


# -------------------------------------------------------- P4 idempotence

@pytest.mark.parametrize("bits", [4, 2, 8])
def test_idempotence(bits):
    """Quantizing the dequantized weights again gives the same bytes for every
    group whose codes reach both 0 and q_max (the dequantized group spans
    exactly q_max steps of the stored scale)."""
    Q = O.qmax(bits)
    g = O.GROUP_SIZE[bits]
    W = S.decode_weight(1, N=64, K=2048)
    q1 = O.quantize_groups(W.reshape(-1, g), bits)
    c1 = q1["codes"].astype(np.int64)
    W2 = ((c1 - q1["zero"][:, None]) * q1["scale"].astype(np.float32)[:, None]).astype(np.float32)
    q2 = O.quantize_groups(W2, bits)
    full = (c1.min(axis=1) == 0) & (c1.max(axis=1) == Q)
    # x_max's code is round(hi/S) + round(-lo/S), two roundings: it falls one
    # short of q_max in a fraction of groups that grows with q_max (about
    # q_max times the fp16 scale's relative rounding), a few percent at 8 bits
    assert full.mean() > (0.99 if bits <= 4 else 0.95)
    assert np.array_equal(q2["codes"][full], q1["codes"][full])
    assert np.array_equal(q2["scale"][full].view(np.uint16), q1["scale"][full].view(np.uint16))
    assert np.array_equal(q2["zero"][full], q1["zero"][full])


# ------------------------------------------------- P5/P6 packing and sizes

@pytest.mark.parametrize("bits", [4, 2, 8])
def test_pack_roundtrip_and_density(bits):
    rng = np.random.default_rng(3)
    c = rng.integers(0, O.qmax(bits) + 1, size=(5, 256)).astype(np.uint8)
    words = O.pack(c, bits)
    assert words.shape == (5, 256 * bits // 32)
    assert np.array_equal(O.unpack(words, bits, 256), c)
    # every bit of every word carries a code bit: the distinct codes of a
    # row change every bit position across rows of random codes.
    assert np.bitwise_or.reduce(words.reshape(-1)) == 0xFFFFFFFF
    if bits == 8:
        # one code per byte, lowest k first: the packed bytes are the codes
        assert np.array_equal(words.astype("<u4").view(np.uint8).reshape(5, 256), c)


def test_dense_size_matches_memory_table(golden):
    """Codes take exactly b bits per weight: LLaMA-70B at INT4 is 35 GB and at
    INT2 17.5 GB (Memory Savings table, Low-bit Quantization: Slimming Large
    Models to the Extreme); scale + zero add 3 bytes per group."""
    t = golden["llama70b_weight_gb"]
    for bits, key in [(4, "INT4"), (2, "INT2"), (8, "INT8")]:
        L = O.Layout(K=8192, N=1024, block_n=1024, bits=[bits])
        cb, ns, nz = L.sizes()
        assert cb * 8 == 8192 * 1024 * bits
        assert ns == nz == 8192 * 1024 // O.GROUP_SIZE[bits]
        assert t["params"] * cb / (8192 * 1024) / 1e9 == pytest.approx(t[key])
    L = O.Layout(K=256, N=256, block_n=128, bits=[4, 2])
    cb, ns, _ = L.sizes()
    assert cb == 128 * 256 // 2 + 128 * 256 // 4 and ns == 128 * 2 + 128 * 4
    # a Channel-mix map with an 8-bit block: offsets are prefix sums of the
    # blocks' sizes in map order
    L = O.Layout(K=256, N=384, block_n=128, bits=[8, 2, 4])
    offs = [(cbo, go) for (_, _, _, _, cbo, go) in L.blocks()]
    assert offs == [(0, 0), (128 * 256, 128 * 2), (128 * 256 + 128 * 64, 128 * 2 + 128 * 4)]
    cb, ns, _ = L.sizes()
    assert cb == 128 * 256 + 128 * 64 + 128 * 128 and ns == 128 * 2 + 128 * 4 + 128 * 2


# ---------------------------------------------------- P7 brute-force matmul

def _exact_linear(x_bits, p):
    L = p.layout
    x = [[Fraction(float(v)) for v in row] for row in O.bf16_bits_to_f64(x_bits)]
    out = []
    for m in range(len(x)):
        row = []
        for n in range(L.N):
            blk = n // L.block_n
            c, s, z, b, g = O.block_fields(p, blk)
            r = n - blk * L.block_n
            acc = Fraction(0)
            for k in range(L.K):
                w = (int(c[r, k]) - int(z[r, k // g])) * Fraction(float(s[r, k // g]))
                acc += x[m][k] * w
            row.append(acc)
        out.append(row)
    return out


@pytest.mark.parametrize("M,K,N,block_n,bits", [
    (1, 128, 3, 3, [4]), (3, 256, 5, 5, [4]), (2, 128, 8, 8, [2]), (3, 256, 7, 7, [2]),
    (2, 256, 4, 4, [8]), (2, 256, 256, 128, [4, 2]), (2, 256, 256, 128, [8, 4]),
])
def test_linear_brute_force(M, K, N, block_n, bits):
    """y[m][n] = sum_k x[m][k] * (c - z) * S, the plain definition in exact
    rational arithmetic, against the fp64 oracle (non-square shapes catch a
    transposed operand)."""
    rng = np.random.default_rng(M * 1000 + K + N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    L = O.Layout(K, N, block_n, bits)
    p = O.quantize_pack(W, L)
    x = S.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    cols = list(range(N)) if N <= 8 else [0, 1, 127, 128, 200, 255]
    y = O.linear(x, p)
    Lsub = p
    exact = _exact_linear(x, Lsub) if N <= 8 else None
    if exact is None:
        # two-block Channel-mix case: exact check on a few columns
        x64 = O.bf16_bits_to_f64(x)
        for n in cols:
            blk = n // block_n
            c, s, z, b, g = O.block_fields(p, blk)
            r = n - blk * block_n
            for m in range(M):
                acc = sum(Fraction(float(x64[m, k])) * (int(c[r, k]) - int(z[r, k // g]))
                          * Fraction(float(s[r, k // g])) for k in range(K))
                assert abs(Fraction(float(y[m, n])) - acc) <= Fraction(1, 10 ** 12) * (1 + abs(acc))
        return
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(y[m, n])) - exact[m][n]) <= Fraction(1, 10 ** 12) * (1 + abs(exact[m][n]))


def test_linear_exact_integer_case():
    """x in {-1,0,1} and weights on a power-of-two grid: y is exact in fp64
    and in bf16, equal to an integer dot product computed independently."""
    rng = np.random.default_rng(11)
    M, K, N = 3, 256, 6
    base = rng.integers(-7, 9, size=(N, K)).astype(np.float64)
    # each group spans exactly 15 steps of 2^-6: force min -7 and max 8
    base[:, 0::128] = -7
    base[:, 1::128] = 8
    W = (base * 2.0 ** -6).astype(np.float32)
    L = O.Layout(K, N, N, [4])
    p = O.quantize_pack(W, L)
    assert np.all(p.scales.view(np.float16).astype(np.float64) == 2.0 ** -6)
    xi = rng.integers(-1, 2, size=(M, K))
    x = S.bf16_bits(xi.astype(np.float32))
    y = O.linear(x, p)
    exact = (xi @ base.astype(np.int64).T) * 2.0 ** -6
    assert np.array_equal(y, exact)
    assert np.array_equal(O.bf16_bits_to_f64(O.f64_to_bf16_bits(y)), exact)


# ------------------------------------ data gradient dX = dY . W_hat

@pytest.mark.parametrize("M,K,N,block_n,bits", [
    (1, 128, 3, 3, [4]), (3, 128, 5, 5, [2]), (2, 256, 7, 7, [4]), (2, 256, 256, 128, [4, 2]),
])
def test_linear_dx_brute_force(M, K, N, block_n, bits):
    """dX[m][k] = sum_n dY[m][n] (c - z) S in exact rational arithmetic,
    straight from the packed fields, against the fp64 oracle; N != K keeps a
    transposed weight from passing."""
    rng = np.random.default_rng(M * 7 + K + N)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    p = O.quantize_pack(W, O.Layout(K, N, block_n, bits))
    dy = S.bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    dy64 = O.bf16_bits_to_f64(dy)
    cols = list(range(K)) if N < 8 else [0, 1, 63, 64, 127, 128, 255]
    dx = O.linear_dx(dy, p)
    assert dx.shape == (M, K)
    assert np.array_equal(O.linear_dx(dy, p, cols), dx[:, cols])
    fields = [O.block_fields(p, b) for b in range(N // block_n)]
    for m in range(M):
        for k in cols[:24]:
            acc = Fraction(0)
            for n in range(N):
                c, sc, z, b, g = fields[n // block_n]
                r = n % block_n
                acc += (Fraction(float(dy64[m, n])) * (int(c[r, k]) - int(z[r, k // g]))
                        * Fraction(float(sc[r, k // g])))
            assert abs(Fraction(float(dx[m, k])) - acc) <= Fraction(1, 10 ** 12) * (1 + abs(acc))


def test_linear_dx_is_the_adjoint_of_linear():
    """<dY, x . W_hat^T> = <dY . W_hat, x> for any x: the data gradient is the
    transpose of the forward product (Channel-mix, three blocks)."""
    rng = np.random.default_rng(5)
    M, K, N = 4, 256, 384
    W = S.decode_weight(1, N=N, K=K)
    p = O.quantize_pack(W, O.Layout(K, N, 128, [4, 2, 4]))
    x = S.activations(M, K, 17)
    dy = S.bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    lhs = float(np.sum(O.bf16_bits_to_f64(dy) * O.linear(x, p)))
    rhs = float(np.sum(O.linear_dx(dy, p) * O.bf16_bits_to_f64(x)))
    scale = float(np.sum(np.abs(O.bf16_bits_to_f64(dy)) @ np.abs(O.dequant(p).astype(np.float64))
                         * np.abs(O.bf16_bits_to_f64(x))))
    assert abs(lhs - rhs) <= 1e-12 * scale


def test_linear_dx_exact_integer_case():
    """dY in {-1, 0, 1} and weights on a 2^-6 grid: dX is an integer product
    times 2^-6, exact in fp64 and in bf16."""
    rng = np.random.default_rng(12)
    M, K, N = 3, 128, 10
    base = rng.integers(-7, 9, size=(N, K)).astype(np.float64)
    base[:, 0] = -7
    base[:, 1] = 8
    W = (base * 2.0 ** -6).astype(np.float32)
    p = O.quantize_pack(W, O.Layout(K, N, N, [4]))
    assert np.all(p.scales.view(np.float16).astype(np.float64) == 2.0 ** -6)
    di = rng.integers(-1, 2, size=(M, N))
    dy = S.bf16_bits(di.astype(np.float32))
    dx = O.linear_dx(dy, p)
    exact = (di @ base.astype(np.int64)) * 2.0 ** -6
    assert np.array_equal(dx, exact)


# ------------------------------------- KV-cache decode attention

def _kv_case(rng, B, Hq, Hkv, D, tp, tw, bits, scale=1.0):
    q = S.bf16_bits((rng.standard_normal((B, Hq, D)) * scale).astype(np.float32))
    k = (rng.standard_normal((B * tp, Hkv * D)) * scale).astype(np.float32)
    v = rng.standard_normal((B * tp, Hkv * D)).astype(np.float32)
    kp = O.kv_cache_pack(k, bits) if tp else None
    vp = O.kv_cache_pack(v, bits) if tp else None
    kw = S.bf16_bits((rng.standard_normal((B, tw, Hkv, D)) * scale).astype(np.float32))
    vw = S.bf16_bits(rng.standard_normal((B, tw, Hkv, D)).astype(np.float32))
    return q, kp, vp, kw, vw


def test_kv_attention_uniform_scores_give_the_mean():
    """q = 0: every score is 0, softmax is uniform, the output is the plain
    mean of the (dequantized and window) values over all tokens."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, D, tp, tw = 2, 4, 2, 128, 5, 3
    _, kp, vp, kw, vw = _kv_case(rng, B, Hq, Hkv, D, tp, tw, 4)
    q = np.zeros((B, Hq, D), dtype=np.uint16)
    out = O.kv_decode_attention(q, kp, vp, kw, vw, B, Hq, Hkv, D)
    vals = np.concatenate([O.dequant(vp).astype(np.float64).reshape(B, tp, Hkv, D),
                           O.bf16_bits_to_f64(vw).reshape(B, tw, Hkv, D)], axis=1)
    for b in range(B):
        for h in range(Hq):
            want = sum(vals[b, t, h // 2] for t in range(tp + tw)) / (tp + tw)
            assert np.allclose(out[b, h], want, rtol=0, atol=1e-12)
    # the error-bound scale sum_t p_t |v_t| is then the mean magnitude
    out2, absw = O.kv_decode_attention(q, kp, vp, kw, vw, B, Hq, Hkv, D, return_abs=True)
    assert np.array_equal(out2, out)
    for b in range(B):
        for h in range(Hq):
            want = sum(np.abs(vals[b, t, h // 2]) for t in range(tp + tw)) / (tp + tw)
            assert np.allclose(absw[b, h], want, rtol=0, atol=1e-12)


def test_kv_attention_one_dominant_token():
    """A key aligned with q far above the others takes all the weight: the
    output is that token's value (the others weigh below e^-60)."""
    rng = np.random.default_rng(22)
    B, Hq, Hkv, D, tp, tw = 1, 2, 1, 128, 9, 2
    q, kp, vp, kw, vw = _kv_case(rng, B, Hq, Hkv, D, tp, tw, 4, scale=0.05)
    qv = np.zeros((B, Hq, D), dtype=np.float32)
    qv[0, :, 0] = 64.0
    q = S.bf16_bits(qv)
    kwv = O.bf16_bits_to_f64(kw).astype(np.float32).copy()
    kwv[0, 1, 0, 0] = 256.0          # window token 1: score 64*256/sqrt(128) ~ 1448
    kw = S.bf16_bits(kwv)
    out = O.kv_decode_attention(q, kp, vp, kw, vw, B, Hq, Hkv, D)
    want = O.bf16_bits_to_f64(vw)[0, 1, 0]
    for h in range(Hq):
        assert np.allclose(out[0, h], want, rtol=0, atol=1e-12)


def test_kv_attention_matches_torch_sdpa():
    """Against torch's scaled_dot_product_attention in float64 on the same
    dequantized keys and values (key/value heads repeated for the query heads
    they serve), INT4 and INT2, packed part and window."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(23)
    for bits, (B, Hq, Hkv, tp, tw) in [(4, (2, 8, 2, 40, 7)), (2, (1, 4, 4, 65, 0)), (4, (1, 6, 3, 0, 5))]:
        D = 128
        q, kp, vp, kw, vw = _kv_case(rng, B, Hq, Hkv, D, tp, tw, bits)
        out = O.kv_decode_attention(q, kp, vp, kw, vw, B, Hq, Hkv, D)
        keys = [O.bf16_bits_to_f64(kw).reshape(B, tw, Hkv, D)]
        vals = [O.bf16_bits_to_f64(vw).reshape(B, tw, Hkv, D)]
        if tp:
            keys.insert(0, O.dequant(kp).astype(np.float64).reshape(B, tp, Hkv, D))
            vals.insert(0, O.dequant(vp).astype(np.float64).reshape(B, tp, Hkv, D))
        K = torch.from_numpy(np.concatenate(keys, 1)).permute(0, 2, 1, 3)   # B, Hkv, T, D
        V = torch.from_numpy(np.concatenate(vals, 1)).permute(0, 2, 1, 3)
        K = K.repeat_interleave(Hq // Hkv, dim=1).contiguous()
        V = V.repeat_interleave(Hq // Hkv, dim=1).contiguous()
        Q = torch.from_numpy(O.bf16_bits_to_f64(q)).reshape(B, Hq, 1, D)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).reshape(B, Hq, D).numpy()
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_kv_attention_head_mapping():
    """Values constant per key/value head: query head h must return the
    constant of head h // (q_heads / kv_heads) whatever the scores are."""
    rng = np.random.default_rng(24)
    B, Hq, Hkv, D, tp, tw = 1, 8, 2, 128, 6, 2
    q, kp, _, kw, _ = _kv_case(rng, B, Hq, Hkv, D, tp, tw, 4)
    v = np.zeros((tp, Hkv * D), dtype=np.float32)
    v[:, :D] = 3.0
    v[:, D:] = -5.0
    vp = O.kv_cache_pack(v, 4)
    vwv = np.zeros((B, tw, Hkv, D), dtype=np.float32)
    vwv[:, :, 0] = 3.0
    vwv[:, :, 1] = -5.0
    out = O.kv_decode_attention(q, kp, vp, kw, S.bf16_bits(vwv), B, Hq, Hkv, D)
    assert np.allclose(O.dequant(vp)[:, :D], 3.0) and np.allclose(O.dequant(vp)[:, D:], -5.0)
    for h in range(Hq):
        assert np.allclose(out[0, h], 3.0 if h < 4 else -5.0, rtol=0, atol=1e-12)


# ------------------------------------------------------ P8 special cases

def test_channel_mix_uniform_equivalence():
    """A Channel-mix layout whose blocks all have the same width is the
    uniform layout, byte for byte."""
    W = S.decode_weight(0, N=512, K=512)
    for b in (4, 2):
        pu = O.quantize_pack(W, O.Layout(512, 512, 512, [b]))
        pc = O.quantize_pack(W, O.Layout(512, 512, 128, [b] * 4))
        assert np.array_equal(pu.codes, pc.codes)
        assert np.array_equal(pu.scales, pc.scales)
        assert np.array_equal(pu.zeros, pc.zeros)


def test_channel_mix_blocks_are_independent_linears():
    """A two-block Channel-mix linear equals its blocks quantized and applied
    as separate uniform linears (block order, offsets)."""
    W = S.decode_weight(3, N=256, K=256)
    x = S.activations(2, 256, 99)
    p = O.quantize_pack(W, O.Layout(256, 256, 128, [2, 4]))
    p0 = O.quantize_pack(W[:128], O.Layout(256, 128, 128, [2]))
    p1 = O.quantize_pack(W[128:], O.Layout(256, 128, 128, [4]))
    y = O.linear(x, p)
    assert np.array_equal(y[:, :128], O.linear(x, p0))
    assert np.array_equal(y[:, 128:], O.linear(x, p1))


# -------------------------------------- P9 the pages' worked examples

def test_page_affine_examples(golden):
    """Section 2.2 of '大模型量化实战': [-5, 10] over 256 levels gives
    s = 15/255 ~ 0.059; for [0.1, 0.9] the unclamped zero point maps
    Q(0.1) -> 0 and Q(0.9) -> 255."""
    ex = golden["affine_example_scale"]
    q = O.quantize_unclamped_example([ex["x_min"], 3.0, ex["x_max"]], ex["bits"])
    assert abs(float(q["s32"][0]) - ex["scale_approx"]) <= ex["printed_digits_tolerance"]
    assert list(q["codes"][0][[0, 2]]) == [0, 255]
    ex = golden["affine_example_zero_point"]
    q = O.quantize_unclamped_example([ex["x_min"], 0.5, ex["x_max"]], ex["bits"])
    assert int(q["codes"][0][0]) == ex["Q_of_x_min"] and int(q["codes"][0][2]) == ex["Q_of_x_max"]
    assert int(q["zero"][0]) < 0          # the page's own formula needs z outside 0..255 here


# ---------------------------------------------- scale rounding, flags

def _group_with_range(bits, rng_value):
    g = O.GROUP_SIZE[bits]
    v = np.zeros(g, dtype=np.float32)
    v[1] = np.float32(rng_value)
    assert float(v[1]) == rng_value
    return v[None, :]


def test_scale_rounds_half_to_even_in_fp16(golden):
    """The stored scale is fp16 (E5M10, max 65504: section 3.1 Table 1 of the
    low-bit LLM survey review), rounded to nearest even."""
    Q = 15
    cases = [
        (Q * (1 + 2 ** -11), 1.0),                  # tie -> even (down)
        (Q * (1 + 3 * 2 ** -11), 1 + 2 ** -9),      # tie -> even (up)
        (Q * (1 + 2 ** -12), 1.0),                  # below half
        (Q * 3 * 2 ** -26, 2 ** -24),               # subnormal, rounds up to the smallest
        (Q * 2.0 ** -25, 1.0),                      # tie to 0 -> degenerate -> 1.0
        (Q * 65504.0, 65504.0),
    ]
    for rngv, expect in cases:
        q = O.quantize_groups(_group_with_range(4, rngv), 4)
        assert float(q["scale"][0]) == expect, (rngv, q["scale"][0])
        assert q["flags"] == 0
    q = O.quantize_groups(_group_with_range(4, Q * 65520.0), 4)
    assert np.isinf(q["scale"][0]) and q["flags"] == O.FLAG_SCALE_OVERFLOW
    assert golden["fp16_max"]["value"] == 65504


def test_degenerate_and_nonfinite_groups():
    g = 128
    v = np.full((1, g), 0.37, dtype=np.float32)
    q = O.quantize_groups(v, 4)
    assert float(q["scale"][0]) == 1.0 and int(q["zero"][0]) == 0
    assert np.all(q["codes"] == 0) and q["flags"] == 0
    v = np.full((1, g), -2.6, dtype=np.float32)
    q = O.quantize_groups(v, 4)               # z = round(2.6) = 3, c = round(-2.6) + 3 = 0
    assert int(q["zero"][0]) == 3 and np.all(q["codes"] == 0)
    for bad in (np.nan, np.inf, -np.inf):
        v = np.zeros((2, g), dtype=np.float32)
        v[1, 5] = bad
        q = O.quantize_groups(v, 4)
        assert q["flags"] == O.FLAG_NONFINITE
        assert list(q["group_flags"]) == [0, O.FLAG_NONFINITE]


# -------------------------------------------- bf16 rounding used in checks

def test_bf16_rounding_of_results(golden):
    """bf16 keeps 7 stored mantissa bits (section 2.1 of '大模型量化实战');
    round to nearest even, checked on ties and against torch's fp32->bf16
    conversion for fp32-exact values."""
    import torch
    assert golden["bf16_layout"]["bf16_mantissa_bits"] == 7
    one = 1.0
    cases = np.array([one + 2 ** -8, one + 3 * 2 ** -8, one + 2 ** -9, -(one + 2 ** -8), 0.0, 2.0 ** -130,
                      3.3895313892515355e38, 3.40e38])
    out = O.bf16_bits_to_f64(O.f64_to_bf16_bits(cases))
    assert out[0] == 1.0 and out[1] == 1 + 2 ** -6 and out[2] == 1.0 and out[3] == -1.0
    assert out[4] == 0.0 and out[5] == 2.0 ** -130 and out[6] == cases[6] and np.isinf(out[7])
    rng = np.random.default_rng(5)
    a = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16_bits(a.astype(np.float64)), ref)
    # inputs generator rounding agrees too
    assert np.array_equal(S.bf16_bits(a), ref)


def test_compare_linear_metrics():
    y = np.array([[1.0, -2.0, 3.0]])
    r = O.compare_linear(O.f64_to_bf16_bits(y), y)
    assert r["normwise"] == 0.0 and r["match"] == 1.0 and r["max_ulp"] == 0
    yb = O.f64_to_bf16_bits(y)
    yb[0, 1] += 1
    r = O.compare_linear(yb, y)
    assert r["max_ulp"] == 1 and r["match"] == pytest.approx(2 / 3)


# ------------------------------------------ the pins catch planted mistakes

def test_planted_mistakes_are_caught():
    """Copies of the quantizer with one slip each fail the closed-form
    exact-scale check; run on the CPU only."""
    def quant_variant(v, bits, slip):
        v = np.asarray(v, dtype=np.float32)
        qm = np.float32(O.qmax(bits) + (1 if slip == "qmax" else 0))
        lo, hi = v.min(axis=1), v.max(axis=1)
        s16 = ((hi - lo) / qm).astype(np.float16)
        s16 = np.where(s16 == 0, np.float16(1), s16)
        Sv = s16.astype(np.float32)
        z = np.clip(np.rint(-lo / Sv), 0, O.qmax(bits))
        if slip == "range_shift":
            c = np.rint((v - lo[:, None]) / Sv[:, None])
        elif slip == "half_away":
            t = v / Sv[:, None]
            c = np.sign(t) * np.floor(np.abs(t) + 0.5) + z[:, None]
        elif slip == "zero_sign":
            c = np.rint(v / Sv[:, None]) - z[:, None]
        else:
            c = np.rint(v / Sv[:, None]) + z[:, None]
        return np.clip(c, 0, O.qmax(bits)), Sv, z

    rng = np.random.default_rng(1)
    bits, Q = 4, 15
    caught = {}
    for slip in ("qmax", "range_shift", "half_away", "zero_sign"):
        caught[slip] = False
        for _ in range(30):
            S0 = float(np.float16(2.0 ** -7 * (1 + int(rng.integers(0, 1024)) / 1024)))
            ka = int(rng.integers(1, 256 * Q))
            if ka % 256 == 128:
                continue
            ties = [ka + 128 + 256 * n for n in range(-Q, Q) if 0 <= ka + 128 + 256 * n <= 256 * Q][:4]
            us, v = _exact_group(bits, S0, ka, list(rng.integers(0, 256 * Q + 1, size=100)) + ties)
            c, Sv, z = quant_variant(v[None, :], bits, slip)
            zz = rne(Fraction(ka, 256))
            expect = [min(max(rne(Fraction(int(u) - ka, 256)) + zz, 0), Q) for u in us]
            if float(Sv[0]) != S0 or list(c[0].astype(int)) != expect:
                caught[slip] = True
                break
    assert all(caught.values()), caught
