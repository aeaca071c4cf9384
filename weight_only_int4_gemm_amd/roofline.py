"""Algorithmic work of one W4A16 matmul and the MI355X peaks it is priced at.

Pure arithmetic on shapes; no GPU and no library calls.

Byte accounting: the bytes a W4A16 matmul must move at least once -- the
packed codes (half a byte per weight), one FP16 scale per group per output
column, the FP16 activations and the FP16 output:

    bytes(M, K, N, g) = K*N/2 + (K/g)*N*2 + 2*M*K + 2*M*N

Against FP16 weights (2 bytes each) the weight part gives the ideal
speed-up of a weight-bound layer, 2 / (1/2 + 2/128) = 3.879 at g = 128, the
"3.87x ideal" of the MARLIN note (anthology of the SOTA, note 305, "Key
results", paper Figure 1).
"""

from __future__ import annotations

# MI355X published peaks (dense, no sparsity).
HBM_PEAK_BYTES_PER_S = 8.0e12
MFMA_F16_PEAK_FLOPS = 2.5e15
CUS = 256
XCDS = 8


def weight_bytes(K: int, N: int, group: int) -> int:
    """Packed codes plus group scales."""
    return K * N // 2 + (K // group) * N * 2


def algorithmic_bytes(M: int, K: int, N: int, group: int) -> int:
    return weight_bytes(K, N, group) + 2 * M * K + 2 * M * N


def flops(M: int, K: int, N: int) -> int:
    return 2 * M * N * K


def bound(M: int, K: int, N: int, group: int) -> str:
    """'hbm' when moving the bytes takes longer than the MFMA work, else 'mfma'."""
    t_hbm = algorithmic_bytes(M, K, N, group) / HBM_PEAK_BYTES_PER_S
    t_mfma = flops(M, K, N) / MFMA_F16_PEAK_FLOPS
    return "hbm" if t_hbm >= t_mfma else "mfma"


def roofline_seconds(M: int, K: int, N: int, group: int) -> float:
    """Shortest time the peaks allow."""
    return max(algorithmic_bytes(M, K, N, group) / HBM_PEAK_BYTES_PER_S,
               flops(M, K, N) / MFMA_F16_PEAK_FLOPS)
