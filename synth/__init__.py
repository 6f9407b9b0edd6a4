"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and rounds them to the storage dtypes
(BF16 rounding is torch's CPU cast, round to nearest even).  It holds none of
the method's arithmetic: no packing, no dequantisation, no quantisation, no
dot products.  Both the oracle side and the HIP side take their inputs from
here; neither side's code lives here.

Every tensor comes from its own ``numpy`` PCG64 stream keyed by
``SeedSequence([config, layer, matrix, kind])`` so the bytes do not depend on
the order in which tensors are generated.

Workload shapes (the pages' models; sizes in rows x cols = N x K):
  * Qwen3-0.6B-shaped text decoder (turbospark-runtime 0.3.0,
    qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step; Qwen3 0.6B defaults of
    the makima Qwen3-TTS config): hidden 1024, q 2048, kv 1024, intermediate
    3072, vocab 151936, 28 layers, tied LM head.
  * Qwen3-1.7B-shaped decoder: hidden 2048, q 2048, kv 1024, intermediate
    6144, vocab 151936, 28 layers.
  * Whisper-base FFN pair (fuel-transformers 0.19.1,
    lazy_quantized_whisper.rs -- encoder_layer fc1/fc2): 2048x512, 512x2048.
  * Whisper-large layer: d_model 1280, FFN 5120, 32 layers; q/k/v/o
    1280x1280, fc1 5120x1280, fc2 1280x5120.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

# kinds of tensors (last SeedSequence word)
K_CODES, K_SCALES, K_BIASES, K_X, K_WF32 = 1, 2, 3, 4, 5


def rng(config: int, layer: int, matrix: int, kind: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([config, layer, matrix, kind])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round to BF16 (nearest even) via torch's CPU cast; return uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bits to float32 (exact) via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).float().numpy()


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8).tobytes()).hexdigest()


# ---- affine-INT8 g64 triplet -----------------------------------------------

@dataclass
class AffineTriplet:
    """The checkpoint form of one affine linear: U32 codes [rows, cols/4]
    (four u8 codes per word, little-endian), BF16 scales and biases
    [rows, cols/64] as uint16 bits."""
    rows: int
    cols: int
    codes: np.ndarray   # uint32 [rows, cols//4]
    scales: np.ndarray  # uint16 [rows, cols//64]
    biases: np.ndarray  # uint16 [rows, cols//64]


def affine_triplet(rows: int, cols: int, key=(0, 0, 0), scale_range=(1e-3, 1e-2)) -> AffineTriplet:
    """codes uniform u8 0..255; scales uniform in scale_range -> BF16;
    biases BF16(-128 * scale_bf16 + N(0, 1e-4))."""
    c, l, m = key
    g = cols // 64
    codes = rng(c, l, m, K_CODES).integers(0, 256, size=rows * cols, dtype=np.uint8)
    s = rng(c, l, m, K_SCALES).uniform(scale_range[0], scale_range[1], size=(rows, g))
    s_bits = to_bf16_bits(s.astype(np.float32))
    s_val = bf16_bits_to_f32(s_bits).astype(np.float64)
    b = -128.0 * s_val + rng(c, l, m, K_BIASES).normal(0.0, 1e-4, size=(rows, g))
    b_bits = to_bf16_bits(b.astype(np.float32))
    return AffineTriplet(rows, cols, codes.view(np.uint32).reshape(rows, cols // 4),
                         s_bits, b_bits)


def affine_triplet_custom(codes_u8: np.ndarray, scales_f32: np.ndarray,
                          biases_f32: np.ndarray) -> AffineTriplet:
    """Build a triplet from explicit values (used for hand-checked cases)."""
    codes_u8 = np.ascontiguousarray(codes_u8, dtype=np.uint8)
    rows, cols = codes_u8.shape
    return AffineTriplet(rows, cols, codes_u8.view(np.uint32).reshape(rows, cols // 4),
                         to_bf16_bits(scales_f32).reshape(rows, cols // 64),
                         to_bf16_bits(biases_f32).reshape(rows, cols // 64))


def x_bf16(m: int, cols: int, key=(0, 0, 0)) -> np.ndarray:
    """Activations BF16(N(0, 1)) as uint16 bits [m, cols]."""
    c, l, mm = key
    return to_bf16_bits(rng(c, l, mm, K_X).standard_normal((m, cols)).astype(np.float32))


def x_f16(m: int, cols: int, key=(0, 0, 0)) -> np.ndarray:
    """Activations f16(N(0, 1)) as uint16 bits [m, cols] (numpy's rounding
    to nearest even)."""
    c, l, mm = key
    return rng(c, l, mm, K_X).standard_normal((m, cols)).astype(np.float32).astype(
        np.float16).view(np.uint16)


def attention_inputs(heads: int, kv_heads: int, head_dim: int, rows: int, key=(0, 0, 0),
                     f16: bool = True):
    """Decode-attention operands as 16-bit bits (f16, else BF16): q [heads,
    head_dim] and K, V caches [rows, kv_heads, head_dim], entries N(0, 1)
    (the scale of per-head RMS-normed q and k)."""
    c, l, mm = key
    g = rng(c, l, mm, K_X)
    a = [g.standard_normal(shape).astype(np.float32)
         for shape in ((heads, head_dim), (rows, kv_heads, head_dim),
                       (rows, kv_heads, head_dim))]
    if f16:
        return tuple(x.astype(np.float16).view(np.uint16) for x in a)
    return tuple(to_bf16_bits(x) for x in a)


def x_f32(m: int, cols: int, key=(0, 0, 0)) -> np.ndarray:
    """Activations f32 N(0, 1) [m, cols]."""
    c, l, mm = key
    return rng(c, l, mm, K_X).standard_normal((m, cols)).astype(np.float32)


def w_f32(rows: int, cols: int, std: float = 0.02, key=(0, 0, 0)) -> np.ndarray:
    """f32 weights N(0, std) [rows=out_features, cols=in_features]."""
    c, l, m = key
    return rng(c, l, m, K_WF32).normal(0.0, std, size=(rows, cols)).astype(np.float32)


# ---- workload shapes --------------------------------------------------------

@dataclass(frozen=True)
class DecoderSpec:
    name: str
    hidden: int
    q: int
    kv: int
    inter: int
    vocab: int
    layers: int


QWEN3_0_6B = DecoderSpec("qwen3-0.6b", 1024, 2048, 1024, 3072, 151936, 28)
QWEN3_1_7B = DecoderSpec("qwen3-1.7b", 2048, 2048, 1024, 6144, 151936, 28)


def decode_step_matrices(spec: DecoderSpec):
    """Projection GEMVs of one decode step in decoder order, as
    (layer, name, rows, cols, stage).  GEMVs with the same stage number read
    the same input ({q,k,v} and {gate,up}); stages run strictly in order."""
    out = []
    stage = 0
    for layer in range(spec.layers):
        out.append((layer, "q", spec.q, spec.hidden, stage))
        out.append((layer, "k", spec.kv, spec.hidden, stage))
        out.append((layer, "v", spec.kv, spec.hidden, stage))
        stage += 1
        out.append((layer, "o", spec.hidden, spec.q, stage))
        stage += 1
        out.append((layer, "gate", spec.inter, spec.hidden, stage))
        out.append((layer, "up", spec.inter, spec.hidden, stage))
        stage += 1
        out.append((layer, "down", spec.hidden, spec.inter, stage))
        stage += 1
    out.append((spec.layers, "lm_head", spec.vocab, spec.hidden, stage))
    return out


@dataclass(frozen=True)
class Qwen3Spec:
    """Decoder shape and config values of a Qwen3 text model (eps and theta
    as the page's f32 config values)."""
    name: str
    hidden: int
    heads: int
    kv_heads: int
    head_dim: int
    inter: int
    vocab: int
    layers: int
    eps: float = 1e-6
    theta: float = 1e6


QWEN3_0_6B_STEP = Qwen3Spec("qwen3-0.6b", 1024, 16, 8, 128, 3072, 151936, 28)
QWEN3_TINY_STEP = Qwen3Spec("qwen3-tiny", 256, 4, 2, 64, 512, 1000, 2)


def qwen3_model(spec: Qwen3Spec, key: int = 0, layers=None):
    """Random-init weights of a Qwen3 decoder in the page's storage forms:
    per layer the affine triplets q, k, v, o, gate, up, down (scales uniform
    in [1e-4, 1e-3]: weights of about 0.04 rms, as trained int8 layers) and
    BF16 norm weights in_norm, q_norm, k_norm, post_norm ~ N(1, 0.1); the
    final norm; the tied embedding table as a triplet [vocab, hidden]."""
    sr = (1e-4, 1e-3)
    hid, d = spec.hidden, spec.head_dim
    shapes = (("q", spec.heads * d, hid), ("k", spec.kv_heads * d, hid),
              ("v", spec.kv_heads * d, hid), ("o", hid, spec.heads * d),
              ("gate", spec.inter, hid), ("up", spec.inter, hid), ("down", hid, spec.inter))
    norms = (("in_norm", hid), ("q_norm", d), ("k_norm", d), ("post_norm", hid))
    out = []
    for li in range(spec.layers if layers is None else layers):
        L = {}
        for j, (name, rows, cols) in enumerate(shapes):
            L[name] = affine_triplet(rows, cols, key=(20 + key, li, j), scale_range=sr)
        for j, (name, n) in enumerate(norms):
            w = rng(20 + key, li, 16 + j, K_WF32).normal(1.0, 0.1, size=n).astype(np.float32)
            L[name] = to_bf16_bits(w)
        out.append(L)
    fw = rng(20 + key, 9999, 0, K_WF32).normal(1.0, 0.1, size=hid).astype(np.float32)
    embed = affine_triplet(spec.vocab, hid, key=(20 + key, 9999, 1), scale_range=sr)
    return {"layers": out, "final_norm": to_bf16_bits(fw), "embed": embed}


WHISPER_BASE_FFN = [("fc1", 2048, 512), ("fc2", 512, 2048)]
WHISPER_LARGE_LAYER = [("q", 1280, 1280), ("k", 1280, 1280), ("v", 1280, 1280),
                       ("o", 1280, 1280), ("fc1", 5120, 1280), ("fc2", 1280, 5120)]
WHISPER_LARGE_LAYERS = 32
WHISPER_LARGE_FRAMES = 1500
