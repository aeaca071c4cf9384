"""Pins for the CPU oracle: checks against facts other than the oracle itself.

Each test fixes the oracle to something the pages or the mathematics decide:
hand-worked fixtures, an exhaustive comparison with an independent rounding
routine, brute force with exact rational sums, closed forms and invariants.
No GPU is used here.
"""

from __future__ import annotations

import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import w4a16_ref as ref
from synth import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fp16_struct(x: float) -> float:
    """Round a double to float16 with Python's own IEEE half packer (RNE)."""
    try:
        return struct.unpack("<e", struct.pack("<e", x))[0]
    except OverflowError:
        return math.copysign(math.inf, x)


def _fp16_exact(fr: Fraction) -> float:
    """Round an exact rational to float16, ties to even, by integer arithmetic."""
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    a = abs(fr)
    # Exponent e with 2**e <= a < 2**(e+1); float16 normal range e in [-14, 15].
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -14)                    # subnormals share the 2**-14 exponent
    quantum = Fraction(2) ** (e - 10)  # 11 significant bits
    units = a / quantum
    fl = units.numerator // units.denominator
    rem = units - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    value = fl * quantum
    if value >= 65520 or value > 65504:
        return sign * math.inf
    return sign * float(value)


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------

def test_nibble_order_golden():
    """Hand-worked words pin the least-significant-first order along K."""
    rows = []
    with open(os.path.join(GOLDEN, "nibble_order.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                rows.append((int(line[0], 16), [int(v) for v in line[1:]]))
    assert len(rows) >= 5
    Bq = np.array([[w for w, _ in rows]], dtype=np.uint32)   # K=8, N=len(rows)
    q = oracle.unpack_codes(Bq)
    for n, (_, codes) in enumerate(rows):
        assert q[:, n].tolist() == codes
    assert np.array_equal(oracle.pack_codes(q), Bq)


def test_pack_unpack_exhaustive_positions():
    """Every value at every nibble position, alone in its word."""
    words = [v << (4 * i) for i in range(8) for v in range(16)]
    Bq = np.array([words], dtype=np.uint32)
    q = oracle.unpack_codes(Bq)
    for col, (i, v) in enumerate((i, v) for i in range(8) for v in range(16)):
        expect = [0] * 8
        expect[i] = v
        assert q[:, col].tolist() == expect
    assert np.array_equal(oracle.pack_codes(q), Bq)


def test_pack_unpack_random_roundtrip():
    rng = np.random.default_rng(7)
    Bq = rng.integers(0, 2**32, size=(64, 48), dtype=np.uint32)
    assert np.array_equal(oracle.pack_codes(oracle.unpack_codes(Bq)), Bq)
    q = rng.integers(0, 16, size=(256, 40))
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(q)), q)


# ---------------------------------------------------------------------------
# Dequantisation: exhaustive over (code, scale) against an independent
# rounding routine.
# ---------------------------------------------------------------------------

def _all_finite_nonzero_fp16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    keep = np.isfinite(vals) & (vals != 0)
    return vals[keep]


def test_dequant_exhaustive_codes_times_every_fp16_scale():
    """16 codes x all 63,486 finite nonzero FP16 scales of both signs.

    The expected value is the double product ``(q - 8) * s`` (exact: a 4-bit
    integer times an 11-bit significand) rounded once by Python's IEEE half
    packer, a routine that shares nothing with numpy's float16 cast.
    """
    scales = _all_finite_nonzero_fp16()
    assert scales.size == 63486
    K = 128                                 # one group; code of row k is k % 16
    q = np.tile(np.arange(16, dtype=np.uint8), K // 16)[:, None]
    q = np.repeat(q, scales.size, axis=1)
    Bq = oracle.pack_codes(q)
    S = scales[None, :]
    W = oracle.dequant(Bq, S, K)
    got = W[:16, :].astype(np.float64)      # rows 0..15 carry codes 0..15
    svals = scales.astype(np.float64).tolist()
    for code in range(16):
        expect = np.array([_fp16_struct((code - 8) * s) for s in svals])
        row = got[code]
        same = (row == expect) | (np.isnan(row) & np.isnan(expect))
        assert same.all(), f"code {code}: {np.count_nonzero(~same)} mismatches"
        # the sign of a zero result follows the sign of the scale
        if code == 8:
            assert np.array_equal(np.signbit(W[8, :]), np.signbit(scales))


def test_dequant_special_cases():
    s = np.array([[0.01, 0.0123, 3.0, 1000.0]], dtype=np.float16)
    for code, factor in [(8, 0), (0, -8), (9, 1), (7, -1), (10, 2), (6, -2),
                         (12, 4), (4, -4)]:
        Bq = oracle.pack_codes(np.full((128, 4), code))
        W = oracle.dequant(Bq, np.repeat(s, 1, axis=0), 128)
        # multiplying by a power of two (or zero) is exact in float16
        assert np.array_equal(W[0].astype(np.float64),
                              factor * s[0].astype(np.float64))


def test_dequant_group_index():
    """Scale row ``k // group``: a different scale per group lands per group."""
    K, N, g = 512, 16, 128
    q = np.full((K, N), 9)                  # w = +1 * s
    S = np.array([[1.0], [2.0], [4.0], [8.0]], dtype=np.float16) * \
        np.arange(1, N + 1, dtype=np.float16)[None, :]
    W = oracle.dequant(oracle.pack_codes(q), S.astype(np.float16), g)
    for k in range(K):
        assert np.array_equal(W[k], S[k // g])


# ---------------------------------------------------------------------------
# The matmul: brute force with exact rational sums on tiny shapes.
# ---------------------------------------------------------------------------

def _brute_force(A, Bq, S, group):
    """Exact C (Fractions) from first principles, in pure Python."""
    M, K = A.shape
    N = Bq.shape[1]
    w = [[0.0] * N for _ in range(K)]
    for k in range(K):
        for n in range(N):
            code = (int(Bq[k // 8, n]) >> (4 * (k % 8))) & 0xF
            w[k][n] = _fp16_struct((code - 8) * float(S[k // group, n]))
    C = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        a = [Fraction(float(x)) for x in A[m]]
        for n in range(N):
            C[m][n] = sum((a[k] * Fraction(w[k][n]) for k in range(K)), Fraction(0))
    return C


@pytest.mark.parametrize("M,K,N,group,seed", [
    (1, 128, 16, 128, 0), (3, 256, 32, 128, 1), (4, 256, 24, 256, 2),
    (2, 384, 8, 128, 3),
])
def test_gemm_brute_force(M, K, N, group, seed):
    A, Bq, S = make_inputs(M, K, N, group, seed)
    C16, C64 = oracle.gemm(A, Bq, S, group)
    exact = _brute_force(A, Bq, S, group)
    absum = np.abs(A.astype(np.float64)) @ np.abs(oracle.dequant(Bq, S, group).astype(np.float64))
    for m in range(M):
        for n in range(N):
            e = float(exact[m][n])
            assert abs(C64[m, n] - e) <= 1e-13 * absum[m, n] + 1e-300
            # C16 is the exact sum rounded once to float16
            assert float(C16[m, n]) == _fp16_exact(exact[m][n])
    C16_32, _ = oracle.gemm_f32(A, Bq, S, group)
    diff = np.abs(C16_32.astype(np.float64) - C16.astype(np.float64))
    assert diff.max() <= 5e-3 * np.abs(C64).max() + 2.0**-10


def test_gemm_closed_forms():
    """Values worked out by hand.

    All-ones activations over one group of 128 with every code 9 give
    ``C = 128 * fp16(s)``; code 7 gives the negative; code 8 gives 0.
    """
    s = np.float16(0.01)
    S = np.full((1, 16), s, dtype=np.float16)
    A = np.ones((2, 128), dtype=np.float16)
    for word, expect in [(0x99999999, 128 * float(s)), (0x77777777, -128 * float(s)),
                         (0x88888888, 0.0)]:
        Bq = np.full((16, 16), word, dtype=np.uint32)
        C16, C64 = oracle.gemm(A, Bq, S, 128)
        assert np.all(C64 == expect)
        assert np.all(C16.astype(np.float64) == expect)
    # 128 * fp16(0.01) is exact: fp16(0.01) = 1311 * 2**-17
    assert 128 * float(s) == 1311 * 2.0**-10


def test_gemm_all_codes_eight_is_zero():
    A, _, S = make_inputs(5, 512, 64, 128, seed=11)
    Bq = np.full((64, 64), 0x88888888, dtype=np.uint32)
    C16, C64 = oracle.gemm(A, Bq, S, 128)
    assert not np.any(C64) and not np.any(C16.astype(np.float64))


def test_gemm_one_hot_rows_select_weight_rows():
    """``A[m] = 2**p * e_k`` gives ``C[m] = 2**p * W[k]`` bit for bit."""
    K, N = 384, 48
    _, Bq, S = make_inputs(1, K, N, 128, seed=5)
    W = oracle.dequant(Bq, S, 128)
    ks = [0, 1, 7, 8, 127, 128, 200, 383]
    ps = [0, 0, 1, -1, 2, 0, -3, 0]
    A = np.zeros((len(ks), K), dtype=np.float16)
    for m, (k, p) in enumerate(zip(ks, ps)):
        A[m, k] = np.float16(2.0**p)
    C16, _ = oracle.gemm(A, Bq, S, 128)
    for m, (k, p) in enumerate(zip(ks, ps)):
        assert np.array_equal(C16[m], (W[k].astype(np.float64) * 2.0**p).astype(np.float16))


def test_gemm_linear_in_activations():
    """With integer activations every product and sum is exact in float64."""
    rng = np.random.default_rng(3)
    K, N = 256, 32
    _, Bq, S = make_inputs(1, K, N, 128, seed=9)
    A1 = rng.integers(-4, 5, size=(3, K)).astype(np.float16)
    A2 = rng.integers(-4, 5, size=(3, K)).astype(np.float16)
    _, C1 = oracle.gemm(A1, Bq, S, 128)
    _, C2 = oracle.gemm(A2, Bq, S, 128)
    _, C12 = oracle.gemm((A1 + A2).astype(np.float16), Bq, S, 128)
    assert np.array_equal(C12, C1 + C2)
    _, Cn = oracle.gemm((-A1).astype(np.float16), Bq, S, 128)
    assert np.array_equal(Cn, -C1)


def test_group_k_equals_replicated_group_128():
    K, N = 512, 32
    A, Bq, _ = make_inputs(4, K, N, 128, seed=21)
    Sk = np.random.default_rng(1).uniform(0.005, 0.02, (1, N)).astype(np.float16)
    _, Ck = oracle.gemm(A, Bq, Sk, K)
    _, C128 = oracle.gemm(A, Bq, np.repeat(Sk, K // 128, axis=0), 128)
    assert np.array_equal(Ck, C128)


def test_gemm_rectangular_orientation():
    """``A[M][K] . W[K][N]`` and not a transposed product: M != K != N."""
    A, Bq, S = make_inputs(3, 256, 40, 128, seed=4)
    C16, C64 = oracle.gemm(A, Bq, S, 128)
    assert C64.shape == (3, 40)
    exact = _brute_force(A[:1, :], Bq[:, :5], S[:, :5], 128)
    assert np.allclose(C64[0, :5], [float(x) for x in exact[0]], rtol=1e-12, atol=0)


def test_gemm_columns_matches_full():
    A, Bq, S = make_inputs(6, 1024, 96, 128, seed=8)
    _, C64 = oracle.gemm(A, Bq, S, 128, chunk=32)
    cols = [0, 5, 31, 32, 64, 95]
    assert np.array_equal(oracle.gemm_columns(A, Bq, S, 128, cols), C64[:, cols])


# ---------------------------------------------------------------------------
# The permuted layout.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("K,N", [(128, 16), (256, 64), (640, 48)])
def test_repack_is_a_bijection(K, N):
    rng = np.random.default_rng(K + N)
    Bq = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    Bp = oracle.repack(Bq)
    assert Bp.dtype == np.uint32 and Bp.size == K * N // 8
    assert np.array_equal(oracle.unrepack(Bp, K, N), Bq)
    # a permutation of nibbles: the multiset of codes is unchanged
    assert np.array_equal(np.sort(oracle.unpack_codes(Bq).ravel()),
                          np.sort(oracle.unpack_codes(Bp.reshape(-1, 1)).ravel()))


def _mfma16x16x32_model(a_frag, b_frag):
    """The 16x16x32 FP16 matrix instruction, from its operand definition.

    ``a_frag[l]`` holds A[row l % 16][k = 8 * (l // 16) + i], i = 0..7;
    ``b_frag[l]`` holds B[k = 8 * (l // 16) + i][col l % 16].  Returns the
    16 x 16 product in float64.
    """
    Am = np.zeros((16, 32))
    Bm = np.zeros((32, 16))
    for l in range(64):
        for i in range(8):
            Am[l % 16, 8 * (l // 16) + i] = a_frag[l][i]
            Bm[8 * (l // 16) + i, l % 16] = b_frag[l][i]
    return Am @ Bm


def test_repack_feeds_the_matrix_instruction():
    """Consume the permuted words the way a wave does and recover ``A . W``.

    Each lane reads four consecutive words per 16-column block and 128-deep
    block of K, splits each word into four 16-bit pairs by shifting by 4r and
    masking ``0x000F000F`` (pair r = codes 2r, 2r+1), and feeds them to the
    instruction model above, 32 K at a time.
    """
    M, K, N = 16, 256, 32
    A, Bq, S = make_inputs(M, K, N, 128, seed=13)
    Bp = oracle.repack(Bq).reshape(N // 16, K // 128, 64, 4)
    Af = A.astype(np.float64)
    C = np.zeros((M, N))
    for n16 in range(N // 16):
        for kb in range(K // 128):
            for j in range(4):
                k0 = 128 * kb + 32 * j
                a_frag = [[Af[l % 16, k0 + 8 * (l // 16) + i] for i in range(8)]
                          for l in range(64)]
                b_frag = []
                for l in range(64):
                    word = int(Bp[n16, kb, l, j])
                    s = float(S[kb, 16 * n16 + l % 16])
                    vals = []
                    for r in range(4):
                        pair = (word >> (4 * r)) & 0x000F000F
                        for code in (pair & 0xF, pair >> 16):
                            vals.append(_fp16_struct((code - 8) * s))
                    b_frag.append(vals)
                C[:, 16 * n16:16 * n16 + 16] += _mfma16x16x32_model(a_frag, b_frag)
    _, C64 = oracle.gemm(A, Bq, S, 128)
    assert np.allclose(C, C64, rtol=0, atol=1e-9)


# ---------------------------------------------------------------------------
# Byte accounting against the pages' closed form.
# ---------------------------------------------------------------------------

def test_ideal_speedup_matches_byte_accounting():
    from weight_only_int4_gemm_amd import roofline
    vals = {}
    with open(os.path.join(GOLDEN, "ideal_speedup.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                vals[line[0]] = float(line[1])
    g = int(vals["group"])
    K, N = 18432, 73728                     # the page's 72k x 18k layer
    w4 = roofline.weight_bytes(K, N, g)
    f16 = 2 * K * N
    ratio = f16 / w4
    assert math.floor(ratio * 100) / 100 == vals["ideal_speedup"]
    # decode-sized activations barely move the ratio
    assert abs(roofline.algorithmic_bytes(1, K, N, g) / w4 - 1) < 1e-3


# ---------------------------------------------------------------------------
# The fused output operation (bias + activation)
# ---------------------------------------------------------------------------

def test_activation_closed_forms():
    """ReLU and SiLU at points whose values are known in closed form.

    sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4, so SiLU(ln 3) = (3/4) ln 3 and
    SiLU(-ln 3) = -(1/4) ln 3; SiLU(0) = 0; SiLU(x) -> x for large x and
    -> 0 (from below) for very negative x.  A sign slip in the sigmoid
    (x * sigmoid(-x)) would swap 3/4 and 1/4."""
    ln3 = math.log(3.0)
    x = np.array([ln3, -ln3, 0.0, 40.0, -40.0, -800.0, 800.0])
    silu = oracle.activation(x, oracle.ACT_SILU)
    assert silu[0] == pytest.approx(0.75 * ln3, rel=1e-15)
    assert silu[1] == pytest.approx(-0.25 * ln3, rel=1e-15)
    assert silu[2] == 0.0
    assert silu[3] == pytest.approx(40.0, rel=1e-16)
    assert silu[4] == pytest.approx(-40.0 * math.exp(-40.0), rel=1e-14)
    assert silu[5] == 0.0 and math.copysign(1.0, silu[5]) == -1.0   # no overflow, -0
    assert silu[6] == 800.0
    relu = oracle.activation(x, oracle.ACT_RELU)
    assert list(relu) == [ln3, 0.0, 0.0, 40.0, 0.0, 0.0, 800.0]
    assert np.array_equal(oracle.activation(x, oracle.ACT_NONE), x)
    with pytest.raises(ValueError):
        oracle.activation(x, 3)


def test_activation_odd_part_identities():
    """act(x) - act(-x) = x for both ReLU and SiLU (sigmoid(x) + sigmoid(-x)
    = 1), on a dense grid that crosses zero."""
    x = np.linspace(-30.0, 30.0, 6001)
    for act in (oracle.ACT_RELU, oracle.ACT_SILU):
        d = oracle.activation(x, act) - oracle.activation(-x, act)
        assert np.max(np.abs(d - x)) <= 1e-14 * np.max(np.abs(x))
    # SiLU's minimum: about -0.278465 at x about -1.278465
    s = oracle.activation(x, oracle.ACT_SILU)
    assert s.min() == pytest.approx(-0.2784645427610738, abs=1e-6)


def test_fused_without_bias_or_activation_is_the_plain_product():
    A, Bq, S = make_inputs(5, 512, 48, 128, seed=21)
    C16, C64 = oracle.gemm(A, Bq, S, 128)
    F16, Y64, Z64 = oracle.gemm_fused(A, Bq, S, 128)
    assert np.array_equal(Y64, C64) and np.array_equal(Z64, C64)
    assert np.array_equal(F16.view(np.uint16), C16.view(np.uint16))


def test_fused_zero_activations_give_act_of_bias():
    """A = 0: every row of the output is act(bias), exactly."""
    from synth import make_bias
    _, Bq, S = make_inputs(1, 256, 64, 128, seed=22)
    A = np.zeros((3, 256), dtype=np.float16)
    bias = make_bias(64, seed=5)
    b64 = bias.astype(np.float64)
    for act, f in ((oracle.ACT_NONE, lambda v: v), (oracle.ACT_RELU, lambda v: max(v, 0.0)),
                   (oracle.ACT_SILU, lambda v: v / (1.0 + math.exp(-v)))):
        C16, Y64, _ = oracle.gemm_fused(A, Bq, S, 128, bias, act)
        for n in range(64):
            want = f(float(b64[n]))
            assert np.all(Y64[:, n] == pytest.approx(want, rel=1e-15, abs=1e-300))
            assert np.all(C16[:, n].astype(np.float64) == _fp16_struct(float(Y64[0, n])))


def test_fused_one_hot_rows_add_bias_to_weight_rows():
    """Row m of A = e_k: Z[m][n] = W[k][n] + bias[n] (column index of the
    bias, not row index: a transposed bias fails on a non-square case)."""
    from synth import make_bias
    K, N = 384, 40
    _, Bq, S = make_inputs(1, K, N, 128, seed=23)
    W = oracle.dequant(Bq, S, 128).astype(np.float64)
    ks = [0, 5, 200, 383]
    A = np.zeros((len(ks), K), dtype=np.float16)
    A[np.arange(len(ks)), ks] = 1.0
    bias = make_bias(N, seed=6)
    _, _, Z64 = oracle.gemm_fused(A, Bq, S, 128, bias, oracle.ACT_RELU)
    for m, k in enumerate(ks):
        assert np.array_equal(Z64[m], W[k] + bias.astype(np.float64))


@pytest.mark.parametrize("act", [1, 2])
def test_fused_brute_force(act):
    """Exact sums (Fractions) plus bias, activation in Python floats, one
    rounding to FP16 by Python's own half packer."""
    from synth import make_bias
    M, K, N = 2, 256, 24
    A, Bq, S = make_inputs(M, K, N, 128, seed=30 + act)
    bias = make_bias(N, seed=7)
    exact = _brute_force(A, Bq, S, 128)
    C16, Y64, _ = oracle.gemm_fused(A, Bq, S, 128, bias, act)
    for m in range(M):
        for n in range(N):
            z = float(exact[m][n] + Fraction(float(bias[n])))
            y = max(z, 0.0) if act == 1 else z / (1.0 + math.exp(-z))
            assert Y64[m, n] == pytest.approx(y, rel=1e-12, abs=1e-12)
            assert float(C16[m, n]) == _fp16_struct(y)


# ---------------------------------------------------------------------------
# Zero points and BF16
# ---------------------------------------------------------------------------

def _bf16_exact(fr: Fraction) -> float:
    """Round an exact rational to BF16 (8 significant bits, exponent from
    -126, subnormal quantum 2^-133), ties to even, by integer arithmetic."""
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 7)
    units = a / quantum
    fl = units.numerator // units.denominator
    rem = units - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    value = fl * quantum
    if value >= Fraction(2) ** 128:          # past the largest finite BF16
        return sign * math.inf
    return sign * float(value)


def _bits_value(bits):
    return oracle.bf16_to_f64(np.array([bits], dtype=np.uint16))[0]


def test_bf16_rounding_matches_torch():
    """float32 -> BF16 against torch's conversion (round to nearest even), on
    random values and on values built to sit exactly on, just above and just
    below a rounding midpoint, both signs, normals and subnormals."""
    import torch
    rng = np.random.default_rng(3)
    hi = rng.integers(0, 2**16, size=20000, dtype=np.uint32)
    hi = hi[((hi >> 7) & 0xFF) != 0xFF]                 # finite only
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = ((hi[:, None] << np.uint32(16)) | lows[None, :]).ravel()
    rnd = rng.integers(0, 2**32, size=20000, dtype=np.uint32)
    rnd = rnd[((rnd >> 23) & 0xFF) != 0xFF]
    x32 = np.concatenate([bits, rnd]).view(np.float32)
    x32 = x32[np.isfinite(x32) & (np.abs(x32) < 3.3e38)]   # no overflow to inf
    ours = oracle.f64_to_bf16(x32.astype(np.float64))
    ref = torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rounding_exact_rationals():
    """Worked values: ties go to the even neighbour, just-above ties round up,
    subnormals keep the 2^-133 quantum, and float64-only values (between
    float32 neighbours) still round on their exact value."""
    cases = [Fraction(1) + Fraction(1, 2**8), Fraction(1) + Fraction(3, 2**8),
             Fraction(1) + Fraction(1, 2**8) + Fraction(1, 2**40),
             Fraction(-255, 2**7) - Fraction(1, 2**9), Fraction(3, 2**134), Fraction(1, 2**134),
             Fraction(129, 2**133), Fraction(2**8 - 1, 2**8) + Fraction(1, 2**9),
             Fraction(12345, 1000), Fraction(-7, 3)]
    for fr in cases:
        got = _bits_value(oracle.f64_to_bf16(np.array([float(fr)]))[0])
        if float(fr) != fr:      # not exact in float64: compare to the float64 value's rounding
            fr = Fraction(float(fr))
        assert got == _bf16_exact(fr), fr


def _scale_sets():
    """A few hundred FP16 and BF16 scales of both signs across the range."""
    rng = np.random.default_rng(11)
    f16 = rng.integers(0, 2**16, size=400, dtype=np.uint16).view(np.float16)
    f16 = f16[np.isfinite(f16) & (f16 != 0)]
    f16 = np.concatenate([f16, np.array([1.0, -1.0, 2.0**-24, 65504.0, 0.0123], np.float16)])
    b16 = rng.integers(0, 2**16, size=400, dtype=np.uint16)
    b16 = b16[((b16 >> 7) & 0xFF) != 0xFF]
    b16 = b16[(b16 & 0x7FFF) != 0]
    b16 = np.concatenate([b16, np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F], np.uint16)])
    return f16, b16


def _codes_zeros_grid(ns):
    """Bq, Z for K = 128, N = ns * 256: column block c holds all 16 codes of
    each of the 16 zero points (q varies along K, z along N)."""
    q = np.tile(np.arange(16), 8)[:, None] * np.ones((1, 256 * ns), dtype=np.int64)
    z = np.tile(np.repeat(np.arange(16), 16), ns)[None, :].astype(np.uint8)
    return oracle.pack_codes(q), z


def test_dequant_awq_fp16_exhaustive_codes_and_zeros():
    f16, _ = _scale_sets()
    Bq, Z = _codes_zeros_grid(1)
    for s in f16:
        S = np.full((1, 256), s, dtype=np.float16)
        W = oracle.dequant_awq(Bq, S, Z, 128, oracle.DTYPE_F16)
        for k in range(16):
            for zz in range(16):
                n = zz * 16 + (k % 16)
                q = k % 16
                want = _fp16_exact((q - zz) * Fraction(float(s)))
                got = float(W[k, n])
                assert got == want or (got == 0 and want == 0), (s, q, zz)


def test_dequant_awq_bf16_exhaustive_codes_and_zeros():
    _, b16 = _scale_sets()
    Bq, Z = _codes_zeros_grid(1)
    for sb in b16:
        S = np.full((1, 256), sb, dtype=np.uint16)
        W = oracle.dequant_awq(Bq, S, Z, 128, oracle.DTYPE_BF16)
        sv = Fraction(float(_bits_value(sb)))
        vals = oracle.bf16_to_f64(W)
        for q in range(16):
            for zz in range(16):
                n = zz * 16 + q
                assert vals[q, n] == _bf16_exact((q - zz) * sv), (hex(sb), q, zz)


def test_dequant_awq_zero_point_eight_is_the_symmetric_format():
    from synth import make_inputs_awq
    A, Bq, S, Z = make_inputs_awq(1, 512, 48, 128, seed=4)
    Z8 = np.full_like(Z, 8)
    W0 = oracle.dequant(Bq, S, 128)
    assert np.array_equal(oracle.dequant_awq(Bq, S, None, 128, 0).view(np.uint16), W0.view(np.uint16))
    assert np.array_equal(oracle.dequant_awq(Bq, S, Z8, 128, 0).view(np.uint16), W0.view(np.uint16))
    _, _, Sb, _ = make_inputs_awq(1, 512, 48, 128, seed=4, bf16=True)
    assert np.array_equal(oracle.dequant_awq(Bq, Sb, None, 128, 1),
                          oracle.dequant_awq(Bq, Sb, Z8, 128, 1))


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("M,K,N,group,seed", [(2, 256, 16, 128, 1), (3, 256, 24, 256, 2)])
def test_gemm_awq_brute_force(dtype, M, K, N, group, seed):
    """Exact rational sums from first principles (codes read bit by bit,
    zero points and scales by index), rounded once by integer arithmetic."""
    from synth import make_inputs_awq
    A, Bq, S, Z = make_inputs_awq(M, K, N, group, seed=seed, bf16=dtype == 1)
    C, C64 = oracle.gemm_awq(A, Bq, S, Z, group, dtype)
    val = (lambda b: Fraction(float(_bits_value(b)))) if dtype else (lambda h: Fraction(float(h)))
    rnd = _bf16_exact if dtype else _fp16_exact
    for m in range(M):
        for n in range(N):
            total = Fraction(0)
            for k in range(K):
                q = (int(Bq[k // 8, n]) >> (4 * (k % 8))) & 0xF
                w = rnd((q - int(Z[k // group, n])) * val(S[k // group, n]))
                total += val(A[m, k]) * Fraction(w)
            got = float(oracle.bf16_to_f64(np.array([C[m, n]]))[0]) if dtype else float(C[m, n])
            assert got == rnd(total), (m, n)
            assert abs(C64[m, n] - float(total)) <= 1e-12 * max(1.0, abs(float(total)))


@pytest.mark.parametrize("dtype", [0, 1])
def test_gemm_awq_codes_at_their_zero_points_give_zero(dtype):
    from synth import make_inputs_awq
    A, _, S, Z = make_inputs_awq(5, 256, 32, 128, seed=9, bf16=dtype == 1)
    q = np.repeat(Z, 128, axis=0)          # every code equals its zero point
    Bq = oracle.pack_codes(q)
    C, C64 = oracle.gemm_awq(A, Bq, S, Z, 128, dtype)
    assert not np.any(C64) and not np.any(oracle.bf16_to_f64(C) if dtype else C.astype(float))


@pytest.mark.parametrize("dtype", [0, 1])
def test_gemm_awq_one_hot_rows_select_weight_rows(dtype):
    from synth import make_inputs_awq
    _, Bq, S, Z = make_inputs_awq(1, 384, 40, 128, seed=12, bf16=dtype == 1)
    W = oracle.dequant_awq(Bq, S, Z, 128, dtype)
    ks = [0, 7, 200, 383]
    one = 0x3F80 if dtype else np.float16(1.0).view(np.uint16)
    A = np.zeros((len(ks), 384), dtype=np.uint16)
    A[np.arange(len(ks)), ks] = one
    if not dtype:
        A = A.view(np.float16)
    C, _ = oracle.gemm_awq(A, Bq, S, Z, 128, dtype)
    for m, k in enumerate(ks):
        assert np.array_equal(C[m].view(np.uint16), W[k].view(np.uint16))


def test_gemm_awq_sampled_columns_match_full():
    from synth import make_inputs_awq
    A, Bq, S, Z = make_inputs_awq(4, 512, 64, 128, seed=13, bf16=True)
    C, C64 = oracle.gemm_awq(A, Bq, S, Z, 128, 1)
    cols = [0, 5, 33, 63]
    Cs, C64s = oracle.gemm_awq(A, Bq, S, Z, 128, 1, cols=cols)
    assert np.array_equal(Cs, C[:, cols]) and np.array_equal(C64s, C64[:, cols])


# ---------------------------------------------------------------------------
# 8-bit weights
# ---------------------------------------------------------------------------

def _golden8():
    canon, perm = [], []
    with open(os.path.join(GOLDEN, "byte_order8.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p = line.split()
            if p[0] == "canonical":
                canon.append((int(p[1], 16), [int(x) for x in p[2:6]]))
            else:
                perm.append(([int(x) for x in p[1:5]], int(p[5], 16)))
    return canon, perm


def test_byte_order8_golden():
    canon, perm = _golden8()
    for word, codes in canon:
        Bq8 = np.array([[word]], dtype=np.uint32)
        assert list(oracle.unpack_codes8(Bq8)[:, 0]) == codes
        assert oracle.pack_codes8(np.array(codes)[:, None])[0, 0] == word
    for codes, word in perm:
        # one column, K = 64: codes k = 0..3 of column 0 are word 0 of lane 0
        q = np.zeros((64, 16), dtype=np.int64)
        q[0:4, 0] = codes
        Bp = oracle.repack8(oracle.pack_codes8(q))
        assert Bp[0] == word, (codes, hex(Bp[0]))


def test_pack_unpack8_roundtrips_and_positions():
    for i in range(4):
        for v in (0, 1, 127, 128, 255):
            q = np.zeros((4, 3), dtype=np.int64)
            q[i, 1] = v
            w = oracle.pack_codes8(q)
            assert w[0, 1] == v << (8 * i) and w[0, 0] == 0
            assert np.array_equal(oracle.unpack_codes8(w), q.astype(np.uint8))
    rng = np.random.default_rng(5)
    B = rng.integers(0, 2**32, size=(64, 48), dtype=np.uint32)
    assert np.array_equal(oracle.pack_codes8(oracle.unpack_codes8(B)), B)


def test_repack8_is_a_bijection():
    rng = np.random.default_rng(6)
    K, N = 192, 48
    B = rng.integers(0, 2**32, size=(K // 4, N), dtype=np.uint32)
    Bp = oracle.repack8(B)
    assert Bp.size == K * N // 4
    assert np.array_equal(oracle.unrepack8(Bp, K, N), B)
    # every code lands in exactly one byte: permuting the codes permutes bytes
    assert np.array_equal(np.sort(Bp.view(np.uint8)), np.sort(B.view(np.uint8).ravel()))


def test_dequant8_codes_times_scales():
    """All 256 codes against 4096 FP16 scales of both signs plus extremes,
    against the exact double product rounded by Python's half packer."""
    rng = np.random.default_rng(7)
    sc = rng.integers(0, 2**16, size=4096, dtype=np.uint16).view(np.float16)
    sc = sc[np.isfinite(sc) & (sc != 0)]
    sc = np.concatenate([sc, np.array([1.0, -1.0, 2**-24, 65504.0, 0.01], np.float16)])
    q = np.repeat(np.arange(256), 1)[:, None] * np.ones((1, sc.size), dtype=np.int64)
    Bq8 = oracle.pack_codes8(q)
    W = oracle.dequant8(Bq8, sc[None, :], 256)
    for ci in range(0, 256, 1):
        row = W[ci]
        for j in range(0, sc.size, 7):          # every 7th scale per code
            want = _fp16_struct((ci - 128) * float(sc[j]))
            got = float(row[j])
            assert got == want or (got == 0 and want == 0), (ci, sc[j])


def test_repack8_feeds_the_matrix_instruction():
    """Consume the permuted 8-bit words the way a wave does and recover
    ``A . W``: per 16-column block and 64-deep block a lane reads words
    4l .. 4l+3; step s of the block takes words 2s and 2s+1, each split by
    a byte mask 0x00FF00FF (codes k, k+1) and the same mask after a shift by
    8 (codes k+2, k+3)."""
    M, K, N = 16, 128, 32
    A, _, S = make_inputs(M, K, N, 128, seed=14)
    Bq8 = np.random.default_rng(15).integers(0, 2**32, size=(K // 4, N), dtype=np.uint32)
    Bp = oracle.repack8(Bq8).reshape(N // 16, K // 64, 64, 4)
    Af = A.astype(np.float64)
    C = np.zeros((M, N))
    for n16 in range(N // 16):
        for kb in range(K // 64):
            for st in range(2):
                k0 = 64 * kb + 32 * st
                a_frag = [[Af[l % 16, k0 + 8 * (l // 16) + i] for i in range(8)]
                          for l in range(64)]
                b_frag = []
                for l in range(64):
                    s = float(S[k0 // 128, 16 * n16 + l % 16])
                    vals = []
                    for j in (2 * st, 2 * st + 1):
                        word = int(Bp[n16, kb, l, j])
                        for pair in (word & 0x00FF00FF, (word >> 8) & 0x00FF00FF):
                            for code in (pair & 0xFF, pair >> 16):
                                vals.append(_fp16_struct((code - 128) * s))
                    b_frag.append(vals)
                C[:, 16 * n16:16 * n16 + 16] += _mfma16x16x32_model(a_frag, b_frag)
    _, C64 = oracle.gemm8(A, Bq8, S, 128)
    assert np.allclose(C, C64, rtol=0, atol=1e-9)


@pytest.mark.parametrize("M,K,N,group,seed", [(2, 128, 16, 128, 1), (3, 256, 24, 128, 2)])
def test_gemm8_brute_force(M, K, N, group, seed):
    A, _, S = make_inputs(M, K, N, group, seed)
    Bq8 = np.random.default_rng(seed + 50).integers(0, 2**32, size=(K // 4, N), dtype=np.uint32)
    C16, C64 = oracle.gemm8(A, Bq8, S, group)
    for m in range(M):
        for n in range(N):
            total = Fraction(0)
            for k in range(K):
                q = (int(Bq8[k // 4, n]) >> (8 * (k % 4))) & 0xFF
                w = _fp16_struct((q - 128) * float(S[k // group, n]))
                total += Fraction(float(A[m, k])) * Fraction(w)
            assert float(C16[m, n]) == _fp16_exact(total)
            assert abs(C64[m, n] - float(total)) <= 1e-12 * max(1.0, abs(float(total)))


def test_gemm8_all_codes_128_is_zero_and_one_hot_rows():
    A, _, S = make_inputs(4, 256, 32, 128, seed=3)
    Bq8 = np.full((64, 32), 0x80808080, dtype=np.uint32)
    assert not np.any(oracle.gemm8(A, Bq8, S, 128)[1])
    Bq8 = np.random.default_rng(4).integers(0, 2**32, size=(64, 32), dtype=np.uint32)
    W = oracle.dequant8(Bq8, S, 128)
    ks = [0, 3, 100, 255]
    A1 = np.zeros((4, 256), dtype=np.float16)
    A1[np.arange(4), ks] = 1.0
    C, _ = oracle.gemm8(A1, Bq8, S, 128)
    for m, k in enumerate(ks):
        assert np.array_equal(C[m].view(np.uint16), W[k].view(np.uint16))


# ---------------------------------------------------------------------------
# 2:4 sparsity
# ---------------------------------------------------------------------------

def test_sparse24_keep_worked_masks():
    """Hand-worked masks: two set bits keep exactly those; more than two keep
    the lowest two; fewer keep only what is set."""
    cases = {0b0011: [1, 1, 0, 0], 0b1010: [0, 1, 0, 1], 0b1100: [0, 0, 1, 1],
             0b1111: [1, 1, 0, 0], 0b1110: [0, 1, 1, 0], 0b0100: [0, 0, 1, 0],
             0b0000: [0, 0, 0, 0], 0b1001: [1, 0, 0, 1], 0xF5: [1, 0, 1, 0]}
    for m, want in cases.items():
        keep = oracle.sparse24_keep(np.array([[m]], dtype=np.uint8))
        assert list(keep[:, 0].astype(int)) == want, bin(m)


def test_dequant_sparse24_zeros_the_pruned_weights():
    from synth import make_inputs
    _, Bq, S = make_inputs(1, 256, 32, 128, seed=40)
    mask = np.random.default_rng(41).integers(0, 16, size=(64, 32)).astype(np.uint8)
    W = oracle.dequant(Bq, S, 128)
    Ws = oracle.dequant_sparse24(Bq, mask, S, 128)
    keep = oracle.sparse24_keep(mask)
    assert keep.sum(axis=0).max() <= 128            # at most two of four
    assert np.array_equal(Ws[keep].view(np.uint16), W[keep].view(np.uint16))
    assert np.all(Ws[~keep].view(np.uint16) == 0)
    assert np.all(keep.reshape(64, 4, 32).sum(axis=1) <= 2)


def test_repack_sparse24_feeds_the_sparse_instruction():
    """Consume the 2:4 words the way a wave does and recover A . W.

    The sparse 16x16x64 instruction, as the hardware computes it: operand S
    (16 x 64) from 64 lanes of eight values and a position word -- lane L
    gives row L % 16, slot i lands at column 16 (L // 16) + 4 (i // 2) + p,
    p = bits 2i..2i+1 of its position word; operand D (64 x 16): lane l gives
    column l % 16, element j at row 32 (j // 8) + 8 (l // 16) + j % 8.  Here
    S is the weights' transposed block (rows = output columns) and D the
    activations' (columns = batch rows), so the result is C transposed."""
    from synth import make_inputs
    M, K, N = 16, 256, 32
    A, Bq, S = make_inputs(M, K, N, 128, seed=42)
    mask = np.random.default_rng(43).integers(0, 16, size=(K // 4, N)).astype(np.uint8)
    Bp = oracle.repack_sparse24(Bq, mask).reshape(N // 16, K // 128, 192)
    Af = A.astype(np.float64)
    Ct = np.zeros((N, M))
    for n16 in range(N // 16):
        for kb in range(K // 128):
            blk = Bp[n16, kb]
            for t in range(2):
                Sm = np.zeros((16, 64))
                for L in range(64):
                    code_word = int(blk[2 * L + t])
                    pos_word = int(blk[128 + L]) >> (16 * t)
                    s = float(S[kb, 16 * n16 + L % 16])
                    for i in range(8):
                        nib = (i >> 1) + ((i & 1) << 2)
                        q = (code_word >> (4 * nib)) & 0xF
                        p = (pos_word >> (2 * i)) & 3
                        Sm[L % 16, 16 * (L // 16) + 4 * (i // 2) + p] += _fp16_struct((q - 8) * s)
                Dm = np.zeros((64, 16))
                for l in range(64):
                    for j in range(16):
                        Dm[32 * (j // 8) + 8 * (l // 16) + j % 8, l % 16] = \
                            Af[l % 16, 128 * kb + 64 * t + 32 * (j // 8) + 8 * (l // 16) + j % 8]
                Ct[16 * n16:16 * n16 + 16, :] += Sm @ Dm
    _, C64 = oracle.gemm_sparse24(A, Bq, mask, S, 128)
    assert np.allclose(Ct.T, C64, rtol=0, atol=1e-9)


@pytest.mark.parametrize("M,K,N,seed", [(2, 128, 16, 1), (3, 256, 16, 2)])
def test_gemm_sparse24_brute_force(M, K, N, seed):
    from synth import make_inputs
    A, Bq, S = make_inputs(M, K, N, 128, seed)
    mask = np.random.default_rng(seed + 60).integers(0, 16, size=(K // 4, N)).astype(np.uint8)
    C16, C64 = oracle.gemm_sparse24(A, Bq, mask, S, 128)
    for m in range(M):
        for n in range(N):
            total = Fraction(0)
            for g in range(K // 4):
                bits = [b for b in range(4) if (int(mask[g, n]) >> b) & 1][:2]
                for b in bits:
                    k = 4 * g + b
                    q = (int(Bq[k // 8, n]) >> (4 * (k % 8))) & 0xF
                    total += Fraction(float(A[m, k])) * Fraction(_fp16_struct((q - 8) * float(S[k // 128, n])))
            assert float(C16[m, n]) == _fp16_exact(total)


def test_gemm_sparse24_empty_mask_is_zero_and_full_mask_keeps_two():
    from synth import make_inputs
    A, Bq, S = make_inputs(4, 256, 32, 128, seed=44)
    zero = np.zeros((64, 32), dtype=np.uint8)
    assert not np.any(oracle.gemm_sparse24(A, Bq, zero, S, 128)[1])
    full = np.full((64, 32), 0xF, dtype=np.uint8)
    two = np.full((64, 32), 0b0011, dtype=np.uint8)
    assert np.array_equal(oracle.gemm_sparse24(A, Bq, full, S, 128)[1],
                          oracle.gemm_sparse24(A, Bq, two, S, 128)[1])
