"""CPU oracle of the quantized frozen base (test infrastructure).

SparseLoRA article §六 (compatibility): SparseLoRA combines with QLoRA, whose
frozen base weights are stored quantized to save memory, and the pair
(SparseQLoRA) keeps that saving while the sparsity removes work.  The pages
name no quantization format.  The reading taken here is the plainest 4-bit
one: each row of a frozen weight is cut into blocks of QBLOCK consecutive
elements; a block holds one fp32 scale s = max|w| / 7 (0 for an all-zero
block) and one signed 4-bit code q = round(w / s) in [-7, 7] per element
(ties to even; w, s and the quotient in fp32), and the layer computes with
the dequantized value q * s in place of w.  So the sparse LoRA layer over a quantized base is the same
masked-dense layer as over a plain base, evaluated at W = dequantize(codes,
scales): the oracle is dequantization (exact in fp64) in front of the
existing forward and backward.

Storage: codes [rows, cols / 2] uint8, element 2j of a row in the low nibble
and 2j + 1 in the high nibble, two's complement; scales [rows, cols / QBLOCK]
fp32.  cols must be a multiple of QBLOCK.
"""
from __future__ import annotations

import numpy as np

__all__ = ["QBLOCK", "quantize_int4_rows", "dequantize_int4_rows", "int4_codes"]

QBLOCK = 64


def quantize_int4_rows(W: np.ndarray, block: int = QBLOCK):
    """Codes and scales of W [rows, cols] (the reading above).  The weight is
    taken as fp32, and the code, an integer decided by floating point, is
    decided in fp32: s = fp32(max|w|) / 7 and q = rint(w / s), both IEEE fp32
    divisions, ties to even."""
    W = np.asarray(W, dtype=np.float32)
    rows, cols = W.shape
    if cols % block:
        raise ValueError("columns must be a multiple of the block")
    Wb = W.reshape(rows, cols // block, block)
    amax = np.abs(Wb).max(axis=2)
    scales = (amax / np.float32(7.0)).astype(np.float32)
    s32 = scales[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (Wb / np.where(s32 > 0, s32, np.float32(1.0))).astype(np.float32)
    q = np.where(s32 > 0, np.rint(quot), np.float32(0.0))
    q = np.clip(q, -7, 7).astype(np.int64).reshape(rows, cols)
    u = (q & 0xF).astype(np.uint8)
    codes = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    return codes, scales


def int4_codes(codes: np.ndarray) -> np.ndarray:
    """The signed 4-bit integers of packed codes [rows, cols / 2] -> [rows, cols]."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = (codes & 0xF).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    q = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.int64)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    return np.where(q >= 8, q - 16, q)


def dequantize_int4_rows(codes: np.ndarray, scales: np.ndarray, block: int = QBLOCK) -> np.ndarray:
    """W = q * s in fp64 (exact: a 4-bit integer times an fp32 scale)."""
    q = int4_codes(codes).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=1)
    return q * s
