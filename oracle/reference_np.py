"""Independent numpy restatement of the oracle, for small shapes only.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).  It exists to
cross-check ``qd_oracle.c`` through a second route: BF16 is decoded by moving
the bits into the top half of a binary32 and viewing it as numpy float32, f16
by numpy's own float16 view, the encoder by vectorised numpy float32 ops.  It
shares no code with the C oracle.

Sources (page title -- section): turbospark-runtime 0.3.0,
src/qwen3_asr_metal.rs -- embed_row_bytes; fuel-transformers 0.19.1,
src/models/lazy_quantized_whisper.rs -- quantize_in_out_to_q4_0.
"""
from __future__ import annotations

import numpy as np

GROUP = 64
QK = 32


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def affine_dense(blob: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Dequantise the whole matrix to f64: w = q * scale + bias."""
    blob = np.asarray(blob, dtype=np.uint8)
    g = cols // GROUP
    codes = blob[: rows * cols].reshape(rows, cols).astype(np.float64)
    sc = blob[rows * cols: rows * cols + rows * g * 2].view(np.uint16).reshape(rows, g)
    bi = blob[rows * cols + rows * g * 2: rows * cols + 2 * rows * g * 2].view(
        np.uint16).reshape(rows, g)
    s = np.repeat(bf16_bits_to_f64(sc), GROUP, axis=1)
    b = np.repeat(bf16_bits_to_f64(bi), GROUP, axis=1)
    return codes * s + b


def q4_0_dense(wq: np.ndarray, rows: int, cols: int) -> np.ndarray:
    nb = rows * cols // QK
    blk = np.asarray(wq, dtype=np.uint8)[: nb * 18].reshape(nb, 18)
    d = blk[:, 0:2].copy().view(np.float16).astype(np.float64).reshape(nb, 1)
    lo = (blk[:, 2:] & 0x0F).astype(np.int64)
    hi = (blk[:, 2:] >> 4).astype(np.int64)
    q = np.concatenate([lo, hi], axis=1)
    return (d * (q - 8)).reshape(rows, cols)


def q4_0_quantize(w: np.ndarray, rows: int, cols: int) -> np.ndarray:
    x = np.asarray(w, dtype=np.float32).reshape(rows * cols // QK, QK)
    idx = np.argmax(np.abs(x), axis=1)  # first index among equal maxima
    mx = x[np.arange(x.shape[0]), idx]
    d = (mx / np.float32(-8.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        id_ = np.where(d != 0, np.float32(1.0) / d, np.float32(0.0)).astype(np.float32)
    t = (x * id_[:, None]).astype(np.float32)
    t = (t + np.float32(8.5)).astype(np.float32)
    q = np.minimum(15, np.trunc(t)).astype(np.uint8)
    out = np.zeros((x.shape[0], 18), dtype=np.uint8)
    out[:, 0:2] = d.astype(np.float16).view(np.uint8).reshape(-1, 2)
    out[:, 2:] = q[:, :16] | (q[:, 16:] << 4)
    stream = out.reshape(-1)
    pad = (-stream.size) % 4
    return np.concatenate([stream, np.zeros(pad, dtype=np.uint8)])


def affine_dense_sub(blob: np.ndarray, rows: int, cols: int, row_sel, col_sel) -> np.ndarray:
    """The dequantised entries w[r, c] = q * scale + bias for the rows
    `row_sel` (all if None) and columns `col_sel`, in f64."""
    blob = np.asarray(blob, dtype=np.uint8)
    g = cols // GROUP
    rs = np.arange(rows) if row_sel is None else np.asarray(row_sel, dtype=np.int64)
    cs = np.asarray(col_sel, dtype=np.int64)
    codes = blob[: rows * cols].reshape(rows, cols)[np.ix_(rs, cs)].astype(np.float64)
    sc = blob[rows * cols: rows * cols + rows * g * 2].view(np.uint16).reshape(rows, g)
    bi = blob[rows * cols + rows * g * 2: rows * cols + 2 * rows * g * 2].view(
        np.uint16).reshape(rows, g)
    s = bf16_bits_to_f64(sc[np.ix_(rs, cs // GROUP)])
    b = bf16_bits_to_f64(bi[np.ix_(rs, cs // GROUP)])
    return codes * s + b
