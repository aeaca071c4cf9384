"""The W4A16 oracle: unpack, dequantise to FP16, matmul, round to FP16.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module.  It shares no code
with the HIP library and imports nothing from it.

Notation (the pages' own): ``A`` are the FP16 activations, tokens x
in-features (``M x K``); ``B`` the INT4 weights, in-features x out-features
(``K x N``), stored as codes ``q`` in 0..15 with one FP16 scale per group of
``group`` consecutive in-features per output column; ``C = A . dequant(B)``
is the FP16 output (``M x N``).

Readings of what the pages leave open (each one is also listed with the
design notes):

1. Zero point.  The pages say the codes come from a GPTQ-style quantiser and
   are turned back into real magnitudes by the group scale; they give no zero
   point.  The reading taken is the symmetric one, ``w = (q - 8) * s``.
2. Canonical packing.  Eight codes per 32-bit word along K; code ``k = 8j + i``
   of column ``n`` is bits ``4i .. 4i+3`` of word ``Bq[j][n]`` (least
   significant nibble first).  The pages only say the kernel's own layout is
   permuted; this is the plain order a quantiser hands over.
3. Scale layout: ``S[K/group][N]`` row-major; ``group`` divides K; ``group ==
   K`` is one scale per output column.
4. Dequantisation rounds once: ``fp16_rne(f32(q - 8) * f32(s))``.  The float32
   product of a 4-bit integer and an 11-bit significand is exact, so this is
   the exact product rounded to FP16 once.
5. Accumulation: the pages allow FP16 or FP32 registers; the workload fixes
   FP32.  The oracle accumulates in float64 (``gemm``), which is closer to the
   exact sum than any FP32 order; ``gemm_f32`` is the FP32-accumulated twin
   used to show that the FP32 rounding order sits far inside the tolerance.
6. Output: the accumulated value rounded once to FP16 (round-to-nearest-even,
   overflow to infinity).
"""

from __future__ import annotations

import numpy as np

# Reading 1: symmetric codes, zero point 8.
ZERO_POINT = 8

# Version of the permuted layout that ``repack``/``unrepack`` describe.
LAYOUT_VERSION = 1

# Position of code i (0..7, along K) of one fragment inside its 32-bit word in
# the permuted layout: codes 2r and 2r+1 go to nibbles r and r+4, so that one
# shift by 4r and one mask keep the pair (2r, 2r+1) in the two 16-bit halves.
_NIBBLE_OF_CODE = (0, 4, 1, 5, 2, 6, 3, 7)


def _check_words(Bq: np.ndarray) -> None:
    if Bq.dtype != np.uint32 or Bq.ndim != 2:
        raise TypeError("Bq must be a 2-D uint32 array [K/8][N]")


# ---------------------------------------------------------------------------
# Packing (reading 2).  "Quant Marlin kernel" explainer, "The architecture:
# every piece explained", top row: eight 4-bit values in each 32-bit word.
# ---------------------------------------------------------------------------

def unpack_codes(Bq: np.ndarray) -> np.ndarray:
    """Codes ``q[K][N]`` (uint8, 0..15) from canonical words ``Bq[K/8][N]``.

    ``q[8j + i][n] = (Bq[j][n] >> 4i) & 0xF``.
    """
    _check_words(Bq)
    K8, N = Bq.shape
    q = np.empty((K8, 8, N), dtype=np.uint8)
    for i in range(8):
        q[:, i, :] = (Bq >> np.uint32(4 * i)) & np.uint32(0xF)
    return q.reshape(K8 * 8, N)


def pack_codes(q: np.ndarray) -> np.ndarray:
    """Canonical words ``Bq[K/8][N]`` from codes ``q[K][N]`` (0..15)."""
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[0] % 8:
        raise ValueError("q must be [K][N] with K a multiple of 8")
    if q.size and (q.min() < 0 or q.max() > 15):
        raise ValueError("codes must lie in 0..15")
    K, N = q.shape
    q8 = q.astype(np.uint32).reshape(K // 8, 8, N)
    Bq = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        Bq |= q8[:, i, :] << np.uint32(4 * i)
    return Bq


# ---------------------------------------------------------------------------
# Dequantisation (readings 1, 3, 4).  "Quant Marlin kernel" explainer, middle
# row: unpack the INT4 codes to FP16 and multiply by the group scale; "End-to-
# end flow": multiply by the relevant group scale to recover FP16 magnitudes.
# ---------------------------------------------------------------------------

def dequant(Bq: np.ndarray, S: np.ndarray, group: int) -> np.ndarray:
    """FP16 weights ``W[K][N] = fp16_rne(f32(q - 8) * f32(S[k // group][n]))``."""
    _check_words(Bq)
    q = unpack_codes(Bq)
    K, N = q.shape
    S = np.asarray(S)
    if S.dtype != np.float16 or S.shape != (K // group, N) or K % group:
        raise ValueError("S must be float16 [K/group][N] with group | K")
    centred = q.astype(np.float32) - np.float32(ZERO_POINT)
    scale_per_k = np.repeat(S.astype(np.float32), group, axis=0)
    return (centred * scale_per_k).astype(np.float16)


# ---------------------------------------------------------------------------
# The matmul (readings 5, 6).  "Quant Marlin kernel" explainer, middle row:
# FP16 weights times FP16 activations with FP16/FP32 accumulation; bottom
# rows: FP16 activations in, FP16 output out.
# ---------------------------------------------------------------------------

def _check_a(A: np.ndarray, K: int) -> None:
    if A.dtype != np.float16 or A.ndim != 2 or A.shape[1] != K:
        raise ValueError("A must be float16 [M][K]")


def gemm(A: np.ndarray, Bq: np.ndarray, S: np.ndarray, group: int,
         chunk: int = 4096):
    """``(C16, C64)``: the float64-accumulated product and its FP16 rounding.

    ``C64[m][n] = sum_k f64(A[m][k]) * f64(W[k][n])`` with ``W = dequant(...)``;
    ``C16 = fp16_rne(C64)``.  Columns are taken ``chunk`` at a time only to
    bound memory; each output element is the same full sum over K.
    """
    _check_words(Bq)
    K = Bq.shape[0] * 8
    N = Bq.shape[1]
    _check_a(A, K)
    A64 = A.astype(np.float64)
    C64 = np.empty((A.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        W = dequant(np.ascontiguousarray(Bq[:, n0:n1]),
                    np.ascontiguousarray(S[:, n0:n1]), group)
        C64[:, n0:n1] = A64 @ W.astype(np.float64)
    return C64.astype(np.float16), C64


def gemm_f32(A: np.ndarray, Bq: np.ndarray, S: np.ndarray, group: int):
    """FP32-accumulated twin: ``fp16_rne(f32(A) @ f32(W))`` (BLAS order)."""
    K = Bq.shape[0] * 8
    _check_a(A, K)
    W = dequant(Bq, S, group)
    C32 = A.astype(np.float32) @ W.astype(np.float32)
    return C32.astype(np.float16), C32


def gemm_columns(A: np.ndarray, Bq: np.ndarray, S: np.ndarray, group: int,
                 cols) -> np.ndarray:
    """Float64 ``C64[:, cols]``, dequantising only the listed columns.

    Used to check sampled outputs of shapes too large for the whole product.
    """
    cols = np.asarray(cols, dtype=np.int64)
    K = Bq.shape[0] * 8
    _check_a(A, K)
    W = dequant(np.ascontiguousarray(Bq[:, cols]),
                np.ascontiguousarray(S[:, cols]), group)
    return A.astype(np.float64) @ W.astype(np.float64)


# ---------------------------------------------------------------------------
# The permuted layout.  "Low-Precision Quantization Kernels in Production"
# (llms.blog), section 1, mechanism 1, and the "Quant Marlin kernel"
# explainer's note on the permuted weight layout: codes are reordered once,
# offline, so that one wide load hands every lane exactly the operand
# fragment the matrix instruction expects.  The order below is this
# library's own, for the 16x16x32 FP16 matrix instruction of gfx950 (lane l
# supplies column l % 16 and eight consecutive K values 8 * (l // 16) .. +7 of
# a 32-deep K step).  Layout version 1:
#
#   code q[k][n] lives in word
#       ((n16 * (K / 128) + kb) * 64 + lane) * 4 + j
#   with n16 = n // 16, kb = k // 128, j = (k % 128) // 32,
#        lane = (n % 16) + 16 * ((k % 32) // 8),
#   at nibble _NIBBLE_OF_CODE[k % 8].
#
# So one 16-byte load per lane covers that lane's column over one whole
# 128-deep block of K (four 32-deep steps), and a wave's 64 lanes read 1 KiB of
# contiguous memory.
# ---------------------------------------------------------------------------

def _check_layout_shape(K: int, N: int) -> None:
    if K % 128 or N % 16 or K <= 0 or N <= 0:
        raise ValueError(f"layout needs K % 128 == 0 and N % 16 == 0 "
                         f"(K={K}, N={N})")


def repack(Bq: np.ndarray) -> np.ndarray:
    """Permuted words (flat uint32, ``K*N/8`` of them) from canonical ``Bq``."""
    _check_words(Bq)
    K = Bq.shape[0] * 8
    N = Bq.shape[1]
    _check_layout_shape(K, N)
    q = unpack_codes(Bq)                       # [K][N], k = 128kb+32j+8lg+i
    q6 = q.reshape(K // 128, 4, 4, 8, N // 16, 16)   # kb, j, lg, i, n16, nl
    frag = q6.transpose(4, 0, 2, 5, 1, 3)            # n16, kb, lg, nl, j, i
    frag = frag.astype(np.uint32)
    words = np.zeros(frag.shape[:-1], dtype=np.uint32)
    for i in range(8):
        words |= frag[..., i] << np.uint32(4 * _NIBBLE_OF_CODE[i])
    return words.reshape(-1)                   # (n16, kb, lane, j) row-major


def unrepack(Bp: np.ndarray, K: int, N: int) -> np.ndarray:
    """Canonical ``Bq[K/8][N]`` from permuted words (inverse of ``repack``)."""
    _check_layout_shape(K, N)
    Bp = np.asarray(Bp, dtype=np.uint32).reshape(N // 16, K // 128, 4, 16, 4)
    frag = np.empty(Bp.shape + (8,), dtype=np.uint8)
    for i in range(8):
        frag[..., i] = (Bp >> np.uint32(4 * _NIBBLE_OF_CODE[i])) & np.uint32(0xF)
    q6 = frag.transpose(1, 4, 2, 5, 0, 3)            # kb, j, lg, i, n16, nl
    return pack_codes(q6.reshape(K, N))


# ---------------------------------------------------------------------------
# The fused output operation.  "Quant Marlin kernel" explainer, section
# "End-to-end flow": the product goes straight on to the next operation -- a
# bias add, an activation -- as if it came from a plain matmul.
#
# Readings (the pages fix none of these):
#  7. The bias is one FP16 value per output column (``bias[N]``), added to
#     the sum; the activation comes after the bias.
#  8. Fusing means one rounding: ``C = fp16_rne(act(sum + bias))``, with no
#     FP16 rounding of the sum in between.
#  9. The pages name no particular activation.  Offered: none, ReLU
#     (``max(x, 0)``) and SiLU (``x * sigmoid(x)``, the activation of the
#     Llama-family feed-forward layers whose shapes the workload uses).
# ---------------------------------------------------------------------------

ACT_NONE, ACT_RELU, ACT_SILU = 0, 1, 2


def activation(x, act: int) -> np.ndarray:
    """``act`` applied elementwise in float64."""
    x = np.asarray(x, dtype=np.float64)
    if act == ACT_NONE:
        return x.copy()
    if act == ACT_RELU:
        return np.where(x > 0.0, x, 0.0)
    if act == ACT_SILU:
        # sigmoid(x) = 1 / (1 + e^-x), taken on the side where the
        # exponential cannot overflow: e^-|x| <= 1 always.
        e = np.exp(-np.abs(x))
        sig = np.where(x >= 0.0, 1.0 / (1.0 + e), e / (1.0 + e))
        return x * sig
    raise ValueError(f"unknown activation {act}")


def epilogue(C64: np.ndarray, bias, act: int) -> np.ndarray:
    """Float64 ``act(C64 + bias)`` (readings 7-9); ``bias`` None is no bias."""
    Z = np.asarray(C64, dtype=np.float64)
    if bias is not None:
        Z = Z + np.asarray(bias, dtype=np.float16).astype(np.float64)[None, :]
    return activation(Z, act)


def gemm_fused(A: np.ndarray, Bq: np.ndarray, S: np.ndarray, group: int, bias=None,
               act: int = ACT_NONE):
    """``(C16, Y64, Z64)``: the pre-activation ``Z64 = C64 + bias``, the
    float64 output ``Y64 = act(Z64)`` and its single FP16 rounding ``C16``."""
    _, C64 = gemm(A, Bq, S, group)
    Z64 = epilogue(C64, bias, ACT_NONE)
    Y64 = activation(Z64, act)
    return Y64.astype(np.float16), Y64, Z64


# ---------------------------------------------------------------------------
# AWQ-style zero points and BF16.  "Low-Precision Quantization Kernels in
# Production" (llms.blog), section 1 on production engines and the table of
# section 5: the same kernel serves GPTQ and AWQ checkpoints; its
# introduction and section 4: FP16 and BF16 activations.
#
# Readings (the pages define neither format):
# 10. An AWQ-style code carries a zero point per group and output column,
#     w = (q - z) * s, with z an unsigned byte (AWQ's are 0..15) stored
#     uint8 [K/group][N] like the scales.  Without zero points z = 8.
# 11. In the BF16 variant A, the scales and C are BF16; the weight is the
#     exact (q - z) * s rounded once to BF16 (round to nearest, ties to
#     even), the sum is exact (float64 here) and rounded once to BF16.
# BF16 values are carried as their raw 16-bit patterns (uint16): numpy has
# no BF16 type.
# ---------------------------------------------------------------------------

DTYPE_F16, DTYPE_BF16 = 0, 1


def bf16_to_f64(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) -> their values as float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 values to BF16, to nearest with ties to even; returns the
    bit patterns (uint16).  Finite inputs only; overflow gives infinity.

    Rounding is done on the exact value, not through float32: BF16 keeps 8
    significant bits, so x = m * 2^e with the integer m scaled to 2^7..2^8,
    and the rest of the significand decides the rounding."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    sign = np.signbit(x)
    a = np.abs(x)
    nz = a > 0
    # exponent of the leading bit; BF16 normals start at 2^-126, below that
    # the quantum stays 2^-133 (subnormals)
    e = np.floor(np.log2(np.where(nz, a, 1.0))).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    e = np.where(np.ldexp(1.0, e) > a, e - 1, e)
    e = np.where(np.ldexp(1.0, e + 1) <= a, e + 1, e)
    e = np.maximum(e, -126)
    q = np.ldexp(a, 7 - e)                    # significand in units of the quantum
    fl = np.floor(q)
    rem = q - fl                              # exact: q has at most 53 bits
    up = (rem > 0.5) | ((rem == 0.5) & (np.fmod(fl, 2) == 1))
    m = (fl + up).astype(np.int64)            # 0 .. 256
    # m == 256 carries into the next binade
    carry = m == 256
    m = np.where(carry, 128, m)
    e = np.where(carry, e + 1, e)
    normal = m >= 128
    exp_field = np.where(normal, e + 127, 0)
    mant = np.where(normal, m - 128, m)       # subnormal: m < 128 at e = -126
    inf = exp_field >= 255
    bits = np.where(inf, 0x7F80, (exp_field << 7) | mant)
    bits = np.where(nz, bits, 0)
    out[...] = bits.astype(np.uint16)
    out |= (sign.astype(np.uint16) << np.uint16(15))
    return out


def dequant_awq(Bq: np.ndarray, S: np.ndarray, Z, group: int, dtype: int) -> np.ndarray:
    """Weights of the AWQ-style formats (readings 10, 11).

    ``S`` is float16 [K/group][N] for DTYPE_F16 and BF16 bits (uint16) for
    DTYPE_BF16; ``Z`` uint8 [K/group][N] or None (z = 8).  Returns float16
    W[K][N] (DTYPE_F16) or BF16 bits uint16 W[K][N] (DTYPE_BF16), each the
    exact (q - z) * s rounded once."""
    q = unpack_codes(Bq).astype(np.float64)
    K = q.shape[0]
    if Z is None:
        z = np.full(q.shape, float(ZERO_POINT))
    else:
        z = np.repeat(np.asarray(Z, dtype=np.uint8).astype(np.float64), group, axis=0)[:K]
    if dtype == DTYPE_F16:
        s = np.repeat(np.asarray(S, dtype=np.float16).astype(np.float64), group, axis=0)[:K]
        # (q - z) has at most 9 bits and s 11: the float64 product is exact;
        # values past the FP16 range round to infinity
        with np.errstate(over="ignore"):
            return ((q - z) * s).astype(np.float16)
    if dtype == DTYPE_BF16:
        s = np.repeat(bf16_to_f64(S), group, axis=0)[:K]
        return f64_to_bf16((q - z) * s)
    raise ValueError(f"unknown dtype {dtype}")


def gemm_awq(A, Bq: np.ndarray, S, Z, group: int, dtype: int, cols=None):
    """``(C, C64)`` of the AWQ-style formats: C64 = the float64 sum of
    A . W (W from ``dequant_awq``), C its single rounding to ``dtype``
    (float16, or BF16 bits).  ``A`` is float16 [M][K] or BF16 bits.  With
    ``cols``, only those output columns (sampled checks of large shapes)."""
    if cols is not None:
        cols = np.asarray(cols, dtype=np.int64)
        Bq = np.ascontiguousarray(Bq[:, cols])
        S = np.ascontiguousarray(np.asarray(S)[:, cols])
        Z = None if Z is None else np.ascontiguousarray(np.asarray(Z)[:, cols])
    W = dequant_awq(Bq, S, Z, group, dtype)
    if dtype == DTYPE_F16:
        A64 = np.asarray(A, dtype=np.float16).astype(np.float64)
        C64 = A64 @ W.astype(np.float64)
        return C64.astype(np.float16), C64
    A64 = bf16_to_f64(A)
    C64 = A64 @ bf16_to_f64(W)
    return f64_to_bf16(C64), C64


# ---------------------------------------------------------------------------
# 8-bit weights.  "Low-Precision Quantization Kernels in Production"
# (llms.blog), section 1 on production engines: the same kernel serves 4-bit
# and 8-bit checkpoints; the table of section 5: INT4 and INT8.
#
# Readings (the pages define no 8-bit format):
# 12. Codes q in 0..255 centred on 128: w = fp16_rne((q - 128) * s), one FP16
#     scale per group of in-features and column, as for 4 bits.
# 13. Canonical packing: four codes per 32-bit word along K, least
#     significant byte first: code k = 4j + i is bits 8i .. 8i+7 of word
#     Bq8[j][n], Bq8 uint32 [K/4][N].
# 14. The permuted layout (this library's own, version 1 for 8 bits): blocks
#     of 16 columns x 64 in-features (1 KiB), column-block-major then along
#     K; in a block, lane l = (n % 16) + 16 * ((k % 32) // 8) owns words
#     4l .. 4l+3, word j = 2 * ((k % 64) // 32) + (k % 8) // 4, and code k
#     sits at byte (0, 2, 1, 3)[k % 4] of its word.  One 16-byte lane piece
#     then holds the lane's operands of two 32-deep steps of the 16x16x32
#     matrix instruction, and a byte mask pairs codes k, k+1 in the two
#     halves of a register.
# ---------------------------------------------------------------------------

ZERO_POINT8 = 128
_BYTE_OF_CODE8 = (0, 2, 1, 3)


def _check_words8(Bq8: np.ndarray) -> None:
    if Bq8.dtype != np.uint32 or Bq8.ndim != 2:
        raise ValueError("Bq8 must be uint32 [K/4][N]")


def unpack_codes8(Bq8: np.ndarray) -> np.ndarray:
    """Codes ``q[K][N]`` (uint8) from canonical words ``Bq8[K/4][N]``."""
    _check_words8(Bq8)
    K4, N = Bq8.shape
    q = np.empty((K4, 4, N), dtype=np.uint8)
    for i in range(4):
        q[:, i, :] = (Bq8 >> np.uint32(8 * i)) & np.uint32(0xFF)
    return q.reshape(K4 * 4, N)


def pack_codes8(q: np.ndarray) -> np.ndarray:
    """Canonical words ``Bq8[K/4][N]`` from codes ``q[K][N]`` (0..255)."""
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[0] % 4:
        raise ValueError("q must be [K][N] with K a multiple of 4")
    if q.min() < 0 or q.max() > 255:
        raise ValueError("codes must be in 0..255")
    K, N = q.shape
    q4 = q.reshape(K // 4, 4, N).astype(np.uint32)
    out = np.zeros((K // 4, N), dtype=np.uint32)
    for i in range(4):
        out |= q4[:, i, :] << np.uint32(8 * i)
    return out


def dequant8(Bq8: np.ndarray, S: np.ndarray, group: int) -> np.ndarray:
    """FP16 weights ``W[K][N] = fp16_rne((q - 128) * s)`` (reading 12)."""
    q = unpack_codes8(Bq8).astype(np.float64)
    K = q.shape[0]
    s = np.repeat(np.asarray(S, dtype=np.float16).astype(np.float64), group, axis=0)[:K]
    # (q - 128) has 8 bits and s 11: the float64 product is exact
    with np.errstate(over="ignore"):
        return ((q - ZERO_POINT8) * s).astype(np.float16)


def gemm8(A: np.ndarray, Bq8: np.ndarray, S: np.ndarray, group: int, cols=None):
    """``(C16, C64)`` for 8-bit weights: the float64 sum of A . W and its
    single FP16 rounding; with ``cols``, only those output columns."""
    if cols is not None:
        cols = np.asarray(cols, dtype=np.int64)
        Bq8 = np.ascontiguousarray(Bq8[:, cols])
        S = np.ascontiguousarray(np.asarray(S)[:, cols])
    W = dequant8(Bq8, S, group)
    C64 = np.asarray(A, dtype=np.float16).astype(np.float64) @ W.astype(np.float64)
    return C64.astype(np.float16), C64


def repack8(Bq8: np.ndarray) -> np.ndarray:
    """Permuted words (flat uint32, K*N/4 of them) from canonical ``Bq8``
    (reading 14)."""
    _check_words8(Bq8)
    K, N = Bq8.shape[0] * 4, Bq8.shape[1]
    if K % 64 or N % 16:
        raise ValueError("K must be a multiple of 64 and N of 16")
    q = unpack_codes8(Bq8).astype(np.uint32)
    out = np.zeros(K * N // 4, dtype=np.uint32)
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    lane = (n % 16) + 16 * ((k % 32) // 8)
    j = 2 * ((k % 64) // 32) + (k % 8) // 4
    word = (((n // 16) * (K // 64) + k // 64) * 64 + lane) * 4 + j
    byte = np.array(_BYTE_OF_CODE8, dtype=np.uint32)[k % 4]
    np.bitwise_or.at(out, word.ravel(), (q << (np.uint32(8) * byte)).ravel())
    return out


def unrepack8(Bp: np.ndarray, K: int, N: int) -> np.ndarray:
    """Canonical ``Bq8[K/4][N]`` from permuted words (inverse of ``repack8``)."""
    Bp = np.asarray(Bp, dtype=np.uint32).ravel()
    if Bp.size != K * N // 4:
        raise ValueError("size mismatch")
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    lane = (n % 16) + 16 * ((k % 32) // 8)
    j = 2 * ((k % 64) // 32) + (k % 8) // 4
    word = (((n // 16) * (K // 64) + k // 64) * 64 + lane) * 4 + j
    byte = np.array(_BYTE_OF_CODE8, dtype=np.uint32)[k % 4]
    q = (Bp[word] >> (np.uint32(8) * byte)) & np.uint32(0xFF)
    return pack_codes8(q)


# ---------------------------------------------------------------------------
# 2:4 structured sparsity (Sparse-MARLIN).  "The anthology of the SOTA"
# (dmarx.github.io), the MARLIN note, section "Key results" (the serving
# benchmark of Figure 15: a Sparse-MARLIN variant beside MARLIN).
#
# Readings (the pages give no format):
# 15. In every group of four consecutive in-features of a column at most two
#     weights are kept; the others are exactly zero.  The input is the dense
#     canonical codes Bq [K/8][N] plus a mask uint8 [K/4][N] whose bits 0..3
#     mark the kept in-features 4g + i.  The two kept positions are the two
#     lowest set bits; with fewer than two bits set the missing slots take
#     the lowest unset positions and code 8 (weight 0); bits beyond the two
#     lowest are ignored.  Kept weights are fp16_rne((q - 8) * s) as before.
# 16. The permuted layout (this library's own, version 1 for 2:4): per block
#     of 16 columns x 128 in-features, 768 bytes: first 64 lanes x 8 bytes of
#     codes, then 64 lanes x 4 bytes of positions.  Lane l = (n % 16) +
#     16 * ((k % 64) // 16) of a block holds, for the 64-deep half t = (k %
#     128) // 64, the eight kept codes of in-features 64t + 16 * (l // 16)
#     .. +15 (two per group of four, ascending) in code word t, slot i at
#     nibble {0,4,1,5,2,6,3,7}[i], and their positions in the group (0..3)
#     at bits 16t + 2i .. +1 of its position word.
# ---------------------------------------------------------------------------

def _kept_positions(mask: np.ndarray):
    """(p0, p1, valid0, valid1) for each group: the two kept positions and
    whether each comes from a set mask bit (reading 15)."""
    m = np.asarray(mask, dtype=np.uint8) & np.uint8(0xF)
    bits = np.stack([(m >> np.uint8(i)) & np.uint8(1) for i in range(4)], axis=-1).astype(bool)
    order = np.argsort(~bits, axis=-1, kind="stable")     # set bits first, ascending
    p0, p1 = order[..., 0], order[..., 1]
    v0 = np.take_along_axis(bits, p0[..., None], -1)[..., 0]
    v1 = np.take_along_axis(bits, p1[..., None], -1)[..., 0]
    lo = np.minimum(p0, p1)
    hi = np.maximum(p0, p1)
    vlo = np.where(p0 < p1, v0, v1)
    vhi = np.where(p0 < p1, v1, v0)
    return lo, hi, vlo, vhi


def sparse24_keep(mask: np.ndarray) -> np.ndarray:
    """Boolean keep[K][N]: the weights that are not pruned (reading 15)."""
    lo, hi, vlo, vhi = _kept_positions(mask)
    G, N = lo.shape
    keep = np.zeros((G, 4, N), dtype=bool)
    gi, ni = np.meshgrid(np.arange(G), np.arange(N), indexing="ij")
    keep[gi, lo, ni] = vlo
    keep[gi, hi, ni] = vhi
    return keep.reshape(G * 4, N)


def dequant_sparse24(Bq: np.ndarray, mask: np.ndarray, S: np.ndarray, group: int) -> np.ndarray:
    """FP16 weights with the pruned ones exactly zero (+0)."""
    W = dequant(Bq, S, group)
    return np.where(sparse24_keep(mask), W, np.float16(0.0)).astype(np.float16)


def gemm_sparse24(A, Bq, mask, S, group: int, cols=None):
    """``(C16, C64)`` of the 2:4-sparse product; with ``cols``, only those
    output columns."""
    if cols is not None:
        cols = np.asarray(cols, dtype=np.int64)
        Bq = np.ascontiguousarray(Bq[:, cols])
        mask = np.ascontiguousarray(np.asarray(mask)[:, cols])
        S = np.ascontiguousarray(np.asarray(S)[:, cols])
    W = dequant_sparse24(Bq, mask, S, group)
    C64 = np.asarray(A, dtype=np.float16).astype(np.float64) @ W.astype(np.float64)
    return C64.astype(np.float16), C64


def repack_sparse24(Bq: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Permuted 2:4 words (flat uint32, K*N*3/32 of them: 192 per block of 16
    columns x 128 in-features) from dense codes and mask (readings 15, 16)."""
    q = unpack_codes(Bq)
    K, N = q.shape
    if K % 128 or N % 16:
        raise ValueError("K must be a multiple of 128 and N of 16")
    lo, hi, vlo, vhi = _kept_positions(mask)          # [K/4][N]
    G = K // 4
    gi = np.arange(G)[:, None]
    ni = np.arange(N)[None, :]
    c_lo = np.where(vlo, q[4 * gi + lo, ni], ZERO_POINT).astype(np.uint32)
    c_hi = np.where(vhi, q[4 * gi + hi, ni], ZERO_POINT).astype(np.uint32)
    KB = K // 128
    out = np.zeros((N // 16) * KB * 192, dtype=np.uint32)
    g = np.arange(G)[:, None] * np.ones((1, N), dtype=np.int64)
    n = np.ones((G, 1), dtype=np.int64) * np.arange(N)[None, :]
    k0 = 4 * g                                  # first in-feature of the group
    base = ((n // 16) * KB + k0 // 128) * 192
    lane = (n % 16) + 16 * ((k0 % 64) // 16)
    t = (k0 % 128) // 64
    slot0 = 2 * ((k0 % 16) // 4)                # slots 2r, 2r+1 of group r of the lane
    nib = np.array([0, 4, 1, 5, 2, 6, 3, 7], dtype=np.uint32)
    code_word = base + 2 * lane + t
    pos_word = base + 128 + lane
    for slot_off, code, pos in ((0, c_lo, lo), (1, c_hi, hi)):
        sl = (slot0 + slot_off).astype(np.int64)
        np.bitwise_or.at(out, code_word.ravel(), (code << (np.uint32(4) * nib[sl])).ravel())
        np.bitwise_or.at(out, pos_word.ravel(),
                         (pos.astype(np.uint32) << (np.uint32(16) * t.astype(np.uint32) +
                                                    np.uint32(2) * sl.astype(np.uint32))).ravel())
    return out
