"""Python binding of libqdecode.so (include/qdecode.h).

Argument marshalling only: every function here forwards torch tensors' device
pointers, the sizes and the current HIP stream to the C entry point of the
same name and turns a non-zero status into ``QDError``.  No step of the
computation runs in Python or PyTorch, and there is no fallback: if the
shared library is missing the first call raises.

Weight formats (see include/qdecode.h):
  * affine-INT8 g64 -- turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs
    (PackedLinear::resident, load_packed_linear, embed_row_bytes);
  * ggml Q4_0 -- fuel-transformers 0.19.1,
    src/models/lazy_quantized_whisper.rs (quantize_in_out_to_q4_0, q_linear).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqdecode.so")

QD_OK, QD_EINVAL, QD_ESHAPE, QD_EALIGN, QD_EDEVICE, QD_EHIP, QD_ESTEP, QD_ESCRATCH = range(8)

# every function declared in include/qdecode.h
EXPORTS = (
    "qd_status_string", "qd_last_hip_error", "qd_version",
    "affine_i8_g64_bytes", "affine_i8_g64_scales_offset",
    "affine_i8_g64_biases_offset", "q4_0_bytes",
    "affine_i8_g64_pack", "qgemv_affine_i8_g64", "qgemv_affine_i8_g64_group",
    "qgemv_q4_0", "qgemv_q4_0_group", "qgemm_q4_0_prefill", "q4_0_quantize",
    "qgemv_affine_i8_g64_step_workspace_bytes", "qgemv_affine_i8_g64_step_plan",
    "qgemv_affine_i8_g64_step_run", "qgemv_affine_i8_g64_step_check",
    "qd_stream_read", "qgemv_affine_i8_g64_f16", "affine_i8_g64_embed_rows",
    "qlinear_q4_0_gemv", "qlinear_q4_0_gemm",
    "attention_decode_workspace_bytes", "attention_decode",
    "rmsnorm_f16", "qk_norm_rope_f16", "silu_mul_f16",
    "qwen3_step_workspace_bytes", "qwen3_step_run", "qwen3_step_check",
    "qwen3_step_workspace_offset", "attention_decode_noalloc",
    "qgemv_q4_0_step_workspace_bytes", "qgemv_q4_0_step_plan", "qgemv_q4_0_step_run",
    "qgemv_q4_0_step_check",
)


class Qwen3Layer(ctypes.Structure):
    """qd_qwen3_layer"""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q", "k", "v", "o", "gate", "up", "down", "in_norm", "q_norm", "k_norm",
                 "post_norm", "k_cache", "v_cache")]


class Qwen3Model(ctypes.Structure):
    """qd_qwen3_model"""
    _fields_ = [("hidden", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("inter", ctypes.c_int64), ("vocab", ctypes.c_int64),
                ("n_layers", ctypes.c_int64), ("capacity", ctypes.c_int64),
                ("eps", ctypes.c_float), ("theta", ctypes.c_float),
                ("layers", ctypes.POINTER(Qwen3Layer)), ("final_norm", ctypes.c_void_p),
                ("embed", ctypes.c_void_p)]


class Q40LinearItem(ctypes.Structure):
    """qd_q4_0_linear_item"""
    _fields_ = [("w_q4_0", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("rows", ctypes.c_int64)]


class AffineGemvOp(ctypes.Structure):
    """qd_affine_gemv_op"""
    _fields_ = [("w_packed", ctypes.c_void_p), ("x_bf16", ctypes.c_void_p),
                ("y_bf16", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("stage", ctypes.c_int64)]


class AffineGemvItem(ctypes.Structure):
    """qd_affine_gemv_item"""
    _fields_ = [("w_packed", ctypes.c_void_p), ("y_bf16", ctypes.c_void_p),
                ("rows", ctypes.c_int64)]


class Q40GemvItem(ctypes.Structure):
    """qd_q4_0_gemv_item"""
    _fields_ = [("w_q4_0", ctypes.c_void_p), ("y", ctypes.c_void_p), ("rows", ctypes.c_int64)]


class StepPlan(ctypes.Structure):
    """qd_step_plan (filled by the library, kept by the caller)"""
    _fields_ = [("workspace", ctypes.c_void_p), ("nwg", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("n_ops", ctypes.c_int32),
                ("n_stages", ctypes.c_int32), ("m", ctypes.c_int32),
                ("magic", ctypes.c_uint32), ("tail", ctypes.c_int32),
                ("tail_w", ctypes.c_void_p), ("tail_x", ctypes.c_void_p),
                ("tail_y", ctypes.c_void_p), ("tail_rows", ctypes.c_int64),
                ("tail_cols", ctypes.c_int64), ("format", ctypes.c_int32),
                ("group", ctypes.c_int32)]


class Q40GemvOp(ctypes.Structure):
    """qd_q4_0_gemv_op"""
    _fields_ = [("w_q4_0", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("stage", ctypes.c_int64)]


class QDError(RuntimeError):
    def __init__(self, fn: str, status: int, hip: int = 0):
        self.status = status
        self.hip_error = hip
        msg = lib().qd_status_string(status).decode()
        if status == QD_EHIP:
            msg += f" (hipError {hip})"
        super().__init__(f"{fn}: {msg}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqdecode.so (built in-tree by build.py); raise if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python quantized_transformer_decode_amd/build.py` "
                "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        L.qd_status_string.argtypes = [I]
        L.qd_status_string.restype = ctypes.c_char_p
        L.qd_last_hip_error.argtypes = []
        L.qd_last_hip_error.restype = I
        L.qd_version.argtypes = []
        L.qd_version.restype = ctypes.c_char_p
        for n in ("affine_i8_g64_bytes", "affine_i8_g64_scales_offset",
                  "affine_i8_g64_biases_offset", "q4_0_bytes"):
            getattr(L, n).argtypes = [I64, I64]
            getattr(L, n).restype = SZ
        L.affine_i8_g64_pack.argtypes = [P, P, P, I64, I64, P, P]
        L.qgemv_affine_i8_g64.argtypes = [P, I64, I64, P, P, I64, P]
        L.qgemv_q4_0.argtypes = [P, I64, I64, P, P, I64, P]
        L.qgemv_affine_i8_g64_group.argtypes = [ctypes.POINTER(AffineGemvItem), I64, I64, P,
                                                I64, P]
        L.qgemv_q4_0_group.argtypes = [ctypes.POINTER(Q40GemvItem), I64, I64, P, I64, P]
        L.qgemm_q4_0_prefill.argtypes = [P, I64, I64, P, P, I64, P]
        L.q4_0_quantize.argtypes = [P, I64, I64, P, P]
        OPS = ctypes.POINTER(AffineGemvOp)
        PLAN = ctypes.POINTER(StepPlan)
        L.qgemv_affine_i8_g64_step_workspace_bytes.argtypes = [OPS, I64, I64]
        L.qgemv_affine_i8_g64_step_workspace_bytes.restype = SZ
        L.qgemv_affine_i8_g64_step_plan.argtypes = [OPS, I64, I64, P, SZ, PLAN, P]
        L.qgemv_affine_i8_g64_step_run.argtypes = [PLAN, P]
        L.qgemv_affine_i8_g64_step_check.argtypes = [PLAN, ctypes.POINTER(ctypes.c_uint32), P]
        QOPS = ctypes.POINTER(Q40GemvOp)
        L.qgemv_q4_0_step_workspace_bytes.argtypes = [QOPS, I64, I64]
        L.qgemv_q4_0_step_workspace_bytes.restype = SZ
        L.qgemv_q4_0_step_plan.argtypes = [QOPS, I64, I64, P, SZ, PLAN, P]
        L.qgemv_q4_0_step_run.argtypes = [PLAN, P]
        L.qgemv_q4_0_step_check.argtypes = [PLAN, ctypes.POINTER(ctypes.c_uint32), P]
        L.qd_stream_read.argtypes = [P, SZ, P, P]
        L.qgemv_affine_i8_g64_f16.argtypes = [P, I64, I64, P, P, I64, P]
        LIN = ctypes.POINTER(Q40LinearItem)
        L.qlinear_q4_0_gemv.argtypes = [LIN, I64, I64, P, I64, ctypes.c_int32, P]
        L.qlinear_q4_0_gemm.argtypes = [LIN, I64, I64, P, I64, ctypes.c_int32, P]
        L.affine_i8_g64_embed_rows.argtypes = [P, I64, I64, ctypes.POINTER(ctypes.c_int64), I64,
                                               P, ctypes.c_int32, P]
        L.attention_decode_workspace_bytes.argtypes = [I64, I64, I64]
        F32 = ctypes.c_float
        L.rmsnorm_f16.argtypes = [P, P, P, I64, F32, P, P]
        L.qk_norm_rope_f16.argtypes = [P, P, P, P, P, I64, I64, I64, F32, F32, P, I64, P, P, P,
                                       P]
        L.silu_mul_f16.argtypes = [P, P, P, I64, P]
        MP = ctypes.POINTER(Qwen3Model)
        L.qwen3_step_workspace_bytes.argtypes = [MP]
        L.qwen3_step_workspace_bytes.restype = SZ
        L.qwen3_step_run.argtypes = [MP, P, SZ, P, P, P, ctypes.c_int32, P]
        L.qwen3_step_check.argtypes = [P, ctypes.POINTER(ctypes.c_uint32), P]
        L.qwen3_step_workspace_offset.argtypes = [MP, ctypes.c_int32]
        L.qwen3_step_workspace_offset.restype = I64
        L.attention_decode_workspace_bytes.restype = I64
        L.attention_decode.argtypes = [P, P, P, I64, I64, I64, I64, I64, ctypes.c_float,
                                       ctypes.c_int32, P, P, SZ, P]
        L.attention_decode_noalloc.argtypes = [P, P, P, I64, I64, I64, I64, I64,
                                               ctypes.c_float, ctypes.c_int32, P, P]
        for n in ("affine_i8_g64_pack", "qgemv_affine_i8_g64", "qgemv_q4_0",
                  "qgemv_affine_i8_g64_group", "qgemv_q4_0_group",
                  "qgemm_q4_0_prefill", "q4_0_quantize", "qgemv_affine_i8_g64_step_plan",
                  "qgemv_affine_i8_g64_step_run", "qgemv_affine_i8_g64_step_check",
                  "qd_stream_read", "qgemv_affine_i8_g64_f16", "affine_i8_g64_embed_rows",
                  "qlinear_q4_0_gemv", "qlinear_q4_0_gemm", "attention_decode",
                  "rmsnorm_f16", "qk_norm_rope_f16", "silu_mul_f16", "qwen3_step_run",
                  "qwen3_step_check", "attention_decode_noalloc", "qgemv_q4_0_step_plan",
                  "qgemv_q4_0_step_run", "qgemv_q4_0_step_check"):
            getattr(L, n).restype = I
        _lib = L
    return _lib


def _ptr(t) -> int:
    return t.data_ptr() if hasattr(t, "data_ptr") else int(t)


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(getattr(stream, "cuda_stream", stream))


def _check(fn: str, status: int) -> None:
    if status != QD_OK:
        raise QDError(fn, status, lib().qd_last_hip_error() if status == QD_EHIP else 0)


# ---- layout helpers ----------------------------------------------------------

def affine_i8_g64_bytes(rows: int, cols: int) -> int:
    return int(lib().affine_i8_g64_bytes(rows, cols))


def affine_i8_g64_scales_offset(rows: int, cols: int) -> int:
    return int(lib().affine_i8_g64_scales_offset(rows, cols))


def affine_i8_g64_biases_offset(rows: int, cols: int) -> int:
    return int(lib().affine_i8_g64_biases_offset(rows, cols))


def q4_0_bytes(rows: int, cols: int) -> int:
    return int(lib().q4_0_bytes(rows, cols))


# ---- entry points ------------------------------------------------------------

def affine_i8_g64_pack(codes_u32, scales_bf16, biases_bf16, rows: int, cols: int,
                       blob, stream=None) -> None:
    _check("affine_i8_g64_pack", lib().affine_i8_g64_pack(
        _ptr(codes_u32), _ptr(scales_bf16), _ptr(biases_bf16), rows, cols,
        _ptr(blob), _stream(stream)))


def qgemv_affine_i8_g64(w_packed, rows: int, cols: int, x_bf16, y_bf16, m: int,
                        stream=None) -> None:
    _check("qgemv_affine_i8_g64", lib().qgemv_affine_i8_g64(
        _ptr(w_packed), rows, cols, _ptr(x_bf16), _ptr(y_bf16), m, _stream(stream)))


def qgemv_affine_i8_g64_f16(w_packed, rows: int, cols: int, x_f16, y_f16, m: int,
                            stream=None) -> None:
    _check("qgemv_affine_i8_g64_f16", lib().qgemv_affine_i8_g64_f16(
        _ptr(w_packed), rows, cols, _ptr(x_f16), _ptr(y_f16), m, _stream(stream)))


def affine_i8_g64_embed_rows(w_packed, rows: int, cols: int, token_ids, out,
                             out_f16: bool = True, stream=None) -> None:
    """token_ids: host sequence of ints (1..16 of them)."""
    ids = (ctypes.c_int64 * len(token_ids))(*[int(t) for t in token_ids])
    _check("affine_i8_g64_embed_rows", lib().affine_i8_g64_embed_rows(
        _ptr(w_packed), rows, cols, ids, len(token_ids), _ptr(out), 1 if out_f16 else 0,
        _stream(stream)))


def _linear_items(items):
    """items: iterable of (w_q4_0, bias or None, y, rows)."""
    items = list(items)
    arr = (Q40LinearItem * len(items))()
    for k, (w, b, y, rows) in enumerate(items):
        arr[k] = Q40LinearItem(_ptr(w), None if b is None else _ptr(b), _ptr(y), rows)
    return arr, len(items)


def qlinear_q4_0_gemv(items, cols: int, x, m: int, gelu: bool = False, stream=None) -> None:
    """items: (w_q4_0, bias or None, y, rows) for each product sharing x."""
    arr, n = _linear_items(items)
    _check("qlinear_q4_0_gemv", lib().qlinear_q4_0_gemv(arr, n, cols, _ptr(x), m,
                                                         1 if gelu else 0, _stream(stream)))


def qlinear_q4_0_gemm(items, cols: int, x_bf16, m: int, gelu: bool = False,
                      stream=None) -> None:
    arr, n = _linear_items(items)
    _check("qlinear_q4_0_gemm", lib().qlinear_q4_0_gemm(arr, n, cols, _ptr(x_bf16), m,
                                                         1 if gelu else 0, _stream(stream)))


def qgemv_q4_0(w_q4_0, rows: int, cols: int, x, y, m: int, stream=None) -> None:
    _check("qgemv_q4_0", lib().qgemv_q4_0(
        _ptr(w_q4_0), rows, cols, _ptr(x), _ptr(y), m, _stream(stream)))


def qgemv_affine_i8_g64_group(items, cols: int, x_bf16, m: int, stream=None) -> None:
    """items: sequence of (w_packed, y_bf16, rows) sharing the input x_bf16."""
    items = list(items)
    arr = (AffineGemvItem * max(1, len(items)))()
    for i, (w, y, rows) in enumerate(items):
        arr[i] = AffineGemvItem(_ptr(w), _ptr(y), rows)
    _check("qgemv_affine_i8_g64_group", lib().qgemv_affine_i8_g64_group(
        arr, len(items), cols, _ptr(x_bf16), m, _stream(stream)))


def qgemv_q4_0_group(items, cols: int, x, m: int, stream=None) -> None:
    """items: sequence of (w_q4_0, y, rows) sharing the input x."""
    items = list(items)
    arr = (Q40GemvItem * max(1, len(items)))()
    for i, (w, y, rows) in enumerate(items):
        arr[i] = Q40GemvItem(_ptr(w), _ptr(y), rows)
    _check("qgemv_q4_0_group", lib().qgemv_q4_0_group(
        arr, len(items), cols, _ptr(x), m, _stream(stream)))


def qgemm_q4_0_prefill(w_q4_0, rows: int, cols: int, x_bf16, y, m: int,
                       stream=None) -> None:
    _check("qgemm_q4_0_prefill", lib().qgemm_q4_0_prefill(
        _ptr(w_q4_0), rows, cols, _ptr(x_bf16), _ptr(y), m, _stream(stream)))


def q4_0_quantize(w, rows: int, cols: int, out, stream=None) -> None:
    _check("q4_0_quantize", lib().q4_0_quantize(
        _ptr(w), rows, cols, _ptr(out), _stream(stream)))


def attention_decode_workspace_bytes(heads: int, kv_heads: int, head_dim: int) -> int:
    return int(lib().attention_decode_workspace_bytes(heads, kv_heads, head_dim))


def attention_decode(q, k_cache, v_cache, heads: int, kv_heads: int, head_dim: int,
                     length: int, kv_start: int, scale: float, out, workspace,
                     workspace_bytes: int, f16: bool = True, stream=None) -> None:
    """Grouped-query decode attention of one token over the cache rows
    [kv_start, length); q/out [heads, head_dim], caches [rows, kv_heads,
    head_dim], all f16 (f16=True) or BF16.  workspace: device, 16-byte
    aligned, attention_decode_workspace_bytes(heads, kv_heads, head_dim)
    bytes for any window."""
    _check("attention_decode", lib().attention_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), heads, kv_heads, head_dim, length, kv_start,
        float(scale), 1 if f16 else 0, _ptr(out), _ptr(workspace), workspace_bytes,
        _stream(stream)))


def attention_decode_noalloc(q, k_cache, v_cache, heads: int, kv_heads: int, head_dim: int,
                             length: int, kv_start: int, scale: float, out, f16: bool = True,
                             stream=None) -> None:
    """attention_decode with the chunk partials in the library's static
    scratch (no workspace argument; nothing is allocated)."""
    _check("attention_decode_noalloc", lib().attention_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), heads, kv_heads, head_dim, length, kv_start,
        float(scale), 1 if f16 else 0, _ptr(out), _stream(stream)))


def rmsnorm_f16(x, delta, w, n: int, eps: float, out, stream=None) -> None:
    """x <- f16(x + delta) when delta is given, then out = f16(rmsnorm(x) * w)."""
    _check("rmsnorm_f16", lib().rmsnorm_f16(
        _ptr(x), None if delta is None else _ptr(delta), _ptr(w), n, float(eps), _ptr(out),
        _stream(stream)))


def qk_norm_rope_f16(q, k_src, v_src, q_norm, k_norm, heads: int, kv_heads: int,
                     head_dim: int, eps: float, theta: float, position, capacity: int, k_cache,
                     v_cache, error_word, stream=None) -> None:
    """Per-head RMSNorm + NeoX RoPE at *position (device int32) of q (in
    place) and of k_src into K cache row *position; V row copied."""
    _check("qk_norm_rope_f16", lib().qk_norm_rope_f16(
        _ptr(q), _ptr(k_src), _ptr(v_src), _ptr(q_norm), _ptr(k_norm), heads, kv_heads,
        head_dim, float(eps), float(theta), _ptr(position), capacity, _ptr(k_cache),
        _ptr(v_cache), _ptr(error_word), _stream(stream)))


def silu_mul_f16(gate, up, out, n: int, stream=None) -> None:
    _check("silu_mul_f16", lib().silu_mul_f16(_ptr(gate), _ptr(up), _ptr(out), n,
                                              _stream(stream)))


def qwen3_model(hidden, heads, kv_heads, head_dim, inter, vocab, capacity, eps, theta,
                layers, final_norm, embed):
    """Build the qd_qwen3_model struct.  layers: list of dicts with the
    device tensors (or addresses) of Qwen3Layer's fields.  The struct holds
    device addresses only: the caller keeps every tensor alive while the
    model is in use (the returned object keeps only the host layer array)."""
    arr = (Qwen3Layer * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = Qwen3Layer(*[_ptr(L[n]) for n, _ in Qwen3Layer._fields_])
    m = Qwen3Model(hidden, heads, kv_heads, head_dim, inter, vocab, len(layers), capacity,
                   eps, theta, arr, _ptr(final_norm), _ptr(embed))
    m._layers = arr
    return m


def qwen3_step_workspace_bytes(model) -> int:
    return int(lib().qwen3_step_workspace_bytes(ctypes.byref(model)))


QWEN3_BUFFERS = {"q": 0, "k": 1, "v": 2, "attn": 3, "opart": 4, "gate": 5, "up": 6,
                 "delta": 7, "xalt": 8, "qrope": 9}


def qwen3_step_workspace_offset(model, buffer: str) -> int:
    """Byte offset of one of the step's scratch rows in its workspace (-1:
    not used for this model)."""
    return int(lib().qwen3_step_workspace_offset(ctypes.byref(model), QWEN3_BUFFERS[buffer]))


def qwen3_step_run(model, workspace, workspace_bytes: int, x, position, logits=None,
                   advance: bool = False, stream=None) -> None:
    """One decoder step of the row x at *position (device int32)."""
    _check("qwen3_step_run", lib().qwen3_step_run(
        ctypes.byref(model), _ptr(workspace), workspace_bytes, _ptr(x), _ptr(position),
        None if logits is None else _ptr(logits), 1 if advance else 0, _stream(stream)))


def qwen3_step_check(workspace, stream=None) -> int:
    """Synchronise, then return and clear the step's error word (0: no error;
    bit 1: a position outside the cache)."""
    bits = ctypes.c_uint32(0)
    st = lib().qwen3_step_check(_ptr(workspace), ctypes.byref(bits), _stream(stream))
    if st == QD_ESTEP:
        return int(bits.value)
    _check("qwen3_step_check", st)
    return 0


def stream_read(buf, nbytes: int, sink, stream=None) -> None:
    """Read nbytes of device memory once (a practical HBM read ceiling; not a
    step of the decode path)."""
    _check("qd_stream_read", lib().qd_stream_read(_ptr(buf), nbytes, _ptr(sink),
                                                  _stream(stream)))


# ---- decode step in one launch -------------------------------------------------

def make_ops(specs):
    """specs: iterable of (w_packed, x_bf16, y_bf16, rows, cols, stage) with
    tensors or raw device addresses -> ctypes array of AffineGemvOp."""
    specs = list(specs)
    arr = (AffineGemvOp * len(specs))()
    for i, (w, x, y, rows, cols, stage) in enumerate(specs):
        arr[i] = AffineGemvOp(_ptr(w), _ptr(x), _ptr(y), rows, cols, stage)
    return arr


def qgemv_affine_i8_g64_step_workspace_bytes(ops, m: int = 1) -> int:
    return int(lib().qgemv_affine_i8_g64_step_workspace_bytes(ops, len(ops), m))


def qgemv_affine_i8_g64_step_plan(ops, m, workspace, workspace_bytes: int,
                                  stream=None) -> StepPlan:
    plan = StepPlan()
    _check("qgemv_affine_i8_g64_step_plan", lib().qgemv_affine_i8_g64_step_plan(
        ops, len(ops), m, _ptr(workspace), workspace_bytes, ctypes.byref(plan),
        _stream(stream)))
    return plan


def qgemv_affine_i8_g64_step_run(plan: StepPlan, stream=None) -> None:
    _check("qgemv_affine_i8_g64_step_run",
           lib().qgemv_affine_i8_g64_step_run(ctypes.byref(plan), _stream(stream)))


def make_q4_0_ops(specs):
    """specs: iterable of (w_q4_0, x_f32, y_f32, rows, cols, stage) with
    tensors or raw device addresses -> ctypes array of Q40GemvOp."""
    specs = list(specs)
    arr = (Q40GemvOp * len(specs))()
    for i, (w, x, y, rows, cols, stage) in enumerate(specs):
        arr[i] = Q40GemvOp(_ptr(w), _ptr(x), _ptr(y), rows, cols, stage)
    return arr


def qgemv_q4_0_step_workspace_bytes(ops, m: int = 1) -> int:
    return int(lib().qgemv_q4_0_step_workspace_bytes(ops, len(ops), m))


def qgemv_q4_0_step_plan(ops, m, workspace, workspace_bytes: int, stream=None) -> StepPlan:
    plan = StepPlan()
    _check("qgemv_q4_0_step_plan", lib().qgemv_q4_0_step_plan(
        ops, len(ops), m, _ptr(workspace), workspace_bytes, ctypes.byref(plan),
        _stream(stream)))
    return plan


def qgemv_q4_0_step_run(plan: StepPlan, stream=None) -> None:
    _check("qgemv_q4_0_step_run", lib().qgemv_q4_0_step_run(ctypes.byref(plan), _stream(stream)))


def qgemv_q4_0_step_check(plan: StepPlan, stream=None) -> int:
    """Synchronise and return the step's error word (raises QDError if set)."""
    bits = ctypes.c_uint32(0)
    st = lib().qgemv_q4_0_step_check(ctypes.byref(plan), ctypes.byref(bits), _stream(stream))
    if st not in (QD_OK, QD_ESTEP):
        _check("qgemv_q4_0_step_check", st)
    if st == QD_ESTEP:
        raise QDError(f"qgemv_q4_0_step_check (error bits {bits.value:#x})", st)
    return bits.value


def qgemv_affine_i8_g64_step_check(plan: StepPlan, stream=None) -> int:
    """Synchronise and return the step's error word (raises QDError if set)."""
    bits = ctypes.c_uint32(0)
    st = lib().qgemv_affine_i8_g64_step_check(ctypes.byref(plan), ctypes.byref(bits),
                                              _stream(stream))
    if st not in (QD_OK, QD_ESTEP):
        _check("qgemv_affine_i8_g64_step_check", st)
    if st == QD_ESTEP:
        raise QDError(f"qgemv_affine_i8_g64_step_check (error bits {bits.value:#x})", st)
    return bits.value
