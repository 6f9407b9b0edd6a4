"""CPU oracle for the dequantize-inside-the-matmul decode path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``quantized_transformer_decode_amd``) and imports
nothing from it.

The arithmetic lives in ``qd_oracle.c`` (IEEE double dot products with a
sequential sum; a step-by-step IEEE single emulation of the Q4_0 encoder).
This module only builds that file with gcc, loads it with ctypes and marshals
numpy arrays.  ``reference_np`` holds an independent numpy restatement used to
cross-check the C code on small shapes.

Sources (page title -- section):
  turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs -- PackedLinear::resident,
      load_packed_linear, embed_row_bytes (affine-INT8 g64 format and dequant).
  fuel-transformers 0.19.1, src/models/lazy_quantized_whisper.rs -- module
      documentation, quantize_in_out_to_q4_0, q_linear (Q4_0 format, bake and
      matmul).
  turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step
      (the decoder step: norms, RoPE, decode attention, SiLU-mul, residuals).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqd_oracle.so")

GROUP = 64
QK = 32
BLOCK_BYTES = 18


def build(force: bool = True) -> str:
    """Compile qd_oracle.c with gcc (no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
            "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
            _SRC, "-o", tmp, "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
        L.qdo_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.qdo_f16_to_f64.restype = D
        L.qdo_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.qdo_bf16_to_f64.restype = D
        L.qdo_f32_to_f16_rne.argtypes = [ctypes.c_float]
        L.qdo_f32_to_f16_rne.restype = ctypes.c_uint16
        for name in ("qdo_affine_scales_offset", "qdo_affine_biases_offset",
                     "qdo_affine_bytes", "qdo_q4_0_bytes"):
            getattr(L, name).argtypes = [I64, I64]
            getattr(L, name).restype = I64
        L.qdo_affine_pack.argtypes = [P, P, P, I64, I64, P]
        L.qdo_affine_pack.restype = None
        L.qdo_affine_weight.argtypes = [P, I64, I64, I64, I64]
        L.qdo_affine_weight.restype = D
        L.qdo_affine_gemv.argtypes = [P, I64, I64, P, ctypes.c_int, I64, P, I64, P, I64, P]
        L.qdo_affine_embed_row.argtypes = [P, I64, I64, I64, ctypes.c_int, P]
        L.qdo_affine_gemv_f64.argtypes = [P, I64, I64, P, P, I64, P]
        L.qdo_affine_gemv_f64.restype = None
        L.qdo_f32_to_bf16_rne.argtypes = [ctypes.c_float]
        L.qdo_f32_to_bf16_rne.restype = ctypes.c_uint16
        L.qdo_affine_gemv.restype = None
        L.qdo_q4_0_weight.argtypes = [P, I64, I64, I64]
        L.qdo_q4_0_weight.restype = D
        L.qdo_q4_0_gemm.argtypes = [P, I64, I64, P, ctypes.c_int, I64, P, I64,
                                    P, I64, P]
        L.qdo_q4_0_gemm.restype = None
        L.qdo_q4_0_quantize.argtypes = [P, I64, I64, P]
        L.qdo_q4_0_quantize.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _sel(sel, n):
    if sel is None:
        return None, n
    a = np.ascontiguousarray(np.asarray(sel, dtype=np.int64))
    return a, a.size


# ---- scalar decoders ------------------------------------------------------

def f16_to_f64(bits: int) -> float:
    return lib().qdo_f16_to_f64(int(bits))


def bf16_to_f64(bits: int) -> float:
    return lib().qdo_bf16_to_f64(int(bits))


def f32_to_f16_rne(x: float) -> int:
    return int(lib().qdo_f32_to_f16_rne(float(np.float32(x))))


# ---- affine-INT8 g64 ------------------------------------------------------

def affine_scales_offset(rows: int, cols: int) -> int:
    return int(lib().qdo_affine_scales_offset(rows, cols))


def affine_biases_offset(rows: int, cols: int) -> int:
    return int(lib().qdo_affine_biases_offset(rows, cols))


def affine_bytes(rows: int, cols: int) -> int:
    return int(lib().qdo_affine_bytes(rows, cols))


def affine_pack(codes_u32: np.ndarray, scales_bf16: np.ndarray,
                biases_bf16: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Concatenate the checkpoint triplet into one resident blob (u8)."""
    codes = np.ascontiguousarray(codes_u32).view(np.uint8).reshape(-1)
    sc = np.ascontiguousarray(scales_bf16).view(np.uint8).reshape(-1)
    bi = np.ascontiguousarray(biases_bf16).view(np.uint8).reshape(-1)
    assert codes.size == rows * cols
    assert sc.size == bi.size == rows * (cols // GROUP) * 2
    out = np.empty(affine_bytes(rows, cols), dtype=np.uint8)
    lib().qdo_affine_pack(_ptr(codes), _ptr(sc), _ptr(bi), rows, cols, _ptr(out))
    return out


def affine_weight(blob: np.ndarray, rows: int, cols: int, r: int, c: int) -> float:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    return float(lib().qdo_affine_weight(_ptr(blob), rows, cols, r, c))


def affine_gemv(blob: np.ndarray, rows: int, cols: int, x_bf16: np.ndarray,
                m_sel=None, row_sel=None, x_f16: bool = False) -> np.ndarray:
    """f64 y[len(m_sel), len(row_sel)] for x [m, cols] given as BF16 bits (or
    f16 bits with x_f16)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16).reshape(-1, cols)
    m = x.shape[0]
    ms, n_m = _sel(m_sel, m)
    rs, n_r = _sel(row_sel, rows)
    if ms is not None:
        assert ms.min(initial=0) >= 0 and ms.max(initial=0) < max(m, 1)
    if rs is not None:
        assert rs.min(initial=0) >= 0 and rs.max(initial=0) < max(rows, 1)
    y = np.zeros((n_m, n_r), dtype=np.float64)
    lib().qdo_affine_gemv(_ptr(blob), rows, cols, _ptr(x), int(bool(x_f16)), m, _ptr(ms),
                          n_m, _ptr(rs), n_r, _ptr(y))
    return y


def affine_embed_row(blob: np.ndarray, rows: int, cols: int, token: int,
                     out_f16: bool = True) -> np.ndarray:
    """The tied-embedding row of `token` as uint16 bits (f16, or BF16)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    assert 0 <= token < rows
    out = np.zeros(cols, dtype=np.uint16)
    lib().qdo_affine_embed_row(_ptr(blob), rows, cols, token, int(bool(out_f16)), _ptr(out))
    return out


def f32_to_bf16_rne(x: float) -> int:
    return int(lib().qdo_f32_to_bf16_rne(x))


# ---- ggml Q4_0 -------------------------------------------------------------

def q4_0_bytes(rows: int, cols: int) -> int:
    return int(lib().qdo_q4_0_bytes(rows, cols))


def q4_0_quantize(w_f32: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """f32 [rows=out, cols=in] -> Q4_0 byte stream including the zero pad."""
    w = np.ascontiguousarray(w_f32, dtype=np.float32).reshape(-1)
    assert w.size == rows * cols and cols % QK == 0
    out = np.empty(q4_0_bytes(rows, cols), dtype=np.uint8)
    lib().qdo_q4_0_quantize(_ptr(w), rows, cols, _ptr(out))
    return out


def q4_0_quantize_in_out(w_in_out: np.ndarray, in_features: int,
                         out_features: int) -> np.ndarray:
    """The bake as the Whisper page states it: the weight arrives as
    [in_features, out_features], is transposed to [out, in], then encoded."""
    w = np.asarray(w_in_out, dtype=np.float32).reshape(in_features, out_features)
    return q4_0_quantize(np.ascontiguousarray(w.T), out_features, in_features)


def q4_0_weight(wq: np.ndarray, cols: int, n: int, k: int) -> float:
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    return float(lib().qdo_q4_0_weight(_ptr(wq), cols, n, k))


def q4_0_gemm(wq: np.ndarray, rows: int, cols: int, x: np.ndarray,
              m_sel=None, row_sel=None) -> np.ndarray:
    """f64 y[len(m_sel), len(row_sel)]; x is float32 [m, cols] or BF16 bits
    (uint16) [m, cols]."""
    wq = np.ascontiguousarray(wq, dtype=np.uint8)
    if x.dtype == np.uint16:
        kind = 1
        xa = np.ascontiguousarray(x).reshape(-1, cols)
    else:
        kind = 0
        xa = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, cols)
    m = xa.shape[0]
    ms, n_m = _sel(m_sel, m)
    rs, n_r = _sel(row_sel, rows)
    if ms is not None:
        assert ms.min(initial=0) >= 0 and ms.max(initial=0) < max(m, 1)
    if rs is not None:
        assert rs.min(initial=0) >= 0 and rs.max(initial=0) < max(rows, 1)
    y = np.zeros((n_m, n_r), dtype=np.float64)
    lib().qdo_q4_0_gemm(_ptr(wq), rows, cols, _ptr(xa), kind, m, _ptr(ms), n_m,
                        _ptr(rs), n_r, _ptr(y))
    return y


def gelu_tanh(v: np.ndarray) -> np.ndarray:
    """The tanh form of GELU, 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))),
    in f64 (the Whisper page applies `gelu_tanh` after fc1 without defining
    it; this is the standard tanh approximation of Hendrycks & Gimpel)."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (v + 0.044715 * v ** 3)))


def q_linear(wq: np.ndarray, rows: int, cols: int, x: np.ndarray, bias=None,
             gelu: bool = False, m_sel=None, row_sel=None) -> np.ndarray:
    """fuel-transformers 0.19.1, lazy_quantized_whisper.rs -- q_linear: the
    Q4_0 product, then the optional f32 bias [rows] broadcast over the token
    rows; then, for fc1 in encoder_layer / decoder_layer, gelu_tanh.  f64."""
    y = q4_0_gemm(wq, rows, cols, x, m_sel=m_sel, row_sel=row_sel)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float32).astype(np.float64).reshape(-1)
        assert b.size == rows
        y = y + (b if row_sel is None else b[np.asarray(row_sel)])[None, :]
    return gelu_tanh(y) if gelu else y


# ---- decode attention --------------------------------------------------------

def attention_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, length: int,
                     scale: float, kv_start: int = 0) -> np.ndarray:
    """turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step
    (encode_attention_decode): one query row per head against the cached
    rows [kv_start, length) of its K/V head, softmax(scale * q.k) v, in f64.
    q [heads, d]; k_cache, v_cache [rows, kv_heads, d] (the cache row of
    position t holds every K/V head); q head h reads K/V head
    h // (heads // kv_heads) (grouped-query attention).  Inputs are float
    arrays (decode stored bits before calling)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k_cache, dtype=np.float64)
    v = np.asarray(v_cache, dtype=np.float64)
    heads, d = q.shape
    kv_heads = k.shape[1]
    assert heads % kv_heads == 0 and k.shape[2] == d and 0 <= kv_start < length <= k.shape[0]
    group = heads // kv_heads
    out = np.zeros((heads, d), dtype=np.float64)
    for h in range(heads):
        j = h // group
        s = scale * (k[kv_start:length, j, :] @ q[h])  # scores of the window
        p = np.exp(s - s.max())
        p /= p.sum()
        out[h] = p @ v[kv_start:length, j, :]
    return out


# ---- the decoder step around the GEMVs ---------------------------------------
#
# turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step:
# every buffer of the step (the residual row x, normed, q, the K/V cache
# rows, attn, delta, gate, up, logits) holds f16; the norm weights are BF16.
# The kernels' internal precision is not on the page: each op here is
# evaluated exactly (f64, exact weights) and its result rounded to f16 once,
# where the page stores it.

def round_f16(v) -> np.ndarray:
    """Nearest-even f16 rounding of f64 values, taken directly from f64
    (numpy's double -> half conversion), returned as f64."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).astype(np.float64)


def f16_bits(v) -> np.ndarray:
    """uint16 bits of values that are already f16 numbers."""
    a = np.asarray(v, dtype=np.float64)
    h = a.astype(np.float16)
    assert np.array_equal(h.astype(np.float64), a, equal_nan=True), "not f16 values"
    return h.view(np.uint16)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """encode_rms_norm_bf16w / _perhead: over the last axis,
    y = x / sqrt(mean(x^2) + eps) * w (per head for a [heads, d] input)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope_neox(x: np.ndarray, position: int, theta: float) -> np.ndarray:
    """encode_rope_neox_subdim with the rotary width equal to head_dim:
    rotate-half RoPE on [..., d]; pair (i, i + d/2) turns by the angle
    position * theta^(-2i/d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    ang = position * np.power(float(theta), -2.0 * np.arange(half, dtype=np.float64) / d)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """encode_silu_mul: silu(gate) * up, silu(g) = g / (1 + e^-g)."""
    g = np.asarray(gate, dtype=np.float64)
    return g / (1.0 + np.exp(-g)) * np.asarray(up, dtype=np.float64)


def affine_gemv_f64(blob: np.ndarray, rows: int, cols: int, x: np.ndarray,
                    row_sel=None) -> np.ndarray:
    """y = W x for one f64 vector (exact weights, f64 sum)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(cols))
    rs, n_r = _sel(row_sel, rows)
    y = np.zeros(n_r, dtype=np.float64)
    lib().qdo_affine_gemv_f64(_ptr(blob), rows, cols, _ptr(x), _ptr(rs), n_r, _ptr(y))
    return y


def qwen3_step(x_row, position: int, model: dict, k_caches, v_caches, f16: bool = True,
               logit_rows=None):
    """Qwen3AsrMetalEngine::step for one input row at `position`, in the
    page's op order; appends the rotated K and the V row of every layer at
    cache row `position` (caches [rows, kv_heads, head_dim] f64 arrays,
    modified in place) and returns (x after the last layer, logits of
    `logit_rows` (all rows if None) or None when model["embed"] is None).

    model: hidden, heads, kv_heads, head_dim, inter, eps, theta (the page's
    f32 config values), layers: list of dicts with affine blobs q, k, v, o,
    gate, up, down and norm weights in_norm, q_norm, k_norm, post_norm (f64
    values of BF16 weights); final_norm; embed (the tied table's blob) and
    vocab.  With f16, every stored buffer is rounded to f16 (the page's
    buffers) and the GEMVs read their f16 inputs; without, nothing is
    rounded (the same maths in f64)."""
    hid, heads, kvh, d = model["hidden"], model["heads"], model["kv_heads"], model["head_dim"]
    inter, eps, theta = model["inter"], model["eps"], model["theta"]
    r = round_f16 if f16 else (lambda v: np.asarray(v, dtype=np.float64))
    scale = float(np.float32(1.0) / np.sqrt(np.float32(d)))  # the page's f32 1/sqrt(d)

    def gemv(blob, rows, cols, v, row_sel=None):
        if f16:
            return affine_gemv(blob, rows, cols, f16_bits(v).reshape(1, cols), row_sel=row_sel,
                               x_f16=True)[0]
        return affine_gemv_f64(blob, rows, cols, v, row_sel=row_sel)

    x = r(x_row)
    for L, kc, vc in zip(model["layers"], k_caches, v_caches):
        normed = r(rms_norm(x, L["in_norm"], eps))
        q = r(gemv(L["q"], heads * d, hid, normed)).reshape(heads, d)
        k = r(gemv(L["k"], kvh * d, hid, normed)).reshape(kvh, d)
        v = r(gemv(L["v"], kvh * d, hid, normed)).reshape(kvh, d)
        q = r(rms_norm(q, L["q_norm"], eps))
        k = r(rms_norm(k, L["k_norm"], eps))
        q = r(rope_neox(q, position, theta))
        k = r(rope_neox(k, position, theta))
        kc[position] = k
        vc[position] = v
        attn = r(attention_decode(q, kc, vc, position + 1, scale))
        delta = r(gemv(L["o"], hid, heads * d, attn.reshape(-1)))
        x = r(x + delta)
        normed = r(rms_norm(x, L["post_norm"], eps))
        gate = r(gemv(L["gate"], inter, hid, normed))
        up = r(gemv(L["up"], inter, hid, normed))
        act = r(silu_mul(gate, up))
        delta = r(gemv(L["down"], hid, inter, act))
        x = r(x + delta)
    if model.get("embed") is None:
        return x, None
    normed = r(rms_norm(x, model["final_norm"], eps))
    logits = r(gemv(model["embed"], model["vocab"], hid, normed, row_sel=logit_rows))
    return x, logits


# ---- tolerance metric -------------------------------------------------------

def normwise_error(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| (0 when both are all zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
