"""Oracle-side form of the synthetic Qwen3 decoders (synth.qwen3_model):
affine blobs packed by the oracle, BF16 norm weights widened to f64."""
from __future__ import annotations

import numpy as np

import oracle
import synth

MATS = ("q", "k", "v", "o", "gate", "up", "down")
NORMS = ("in_norm", "q_norm", "k_norm", "post_norm")


def pack(tr) -> np.ndarray:
    return oracle.affine_pack(tr.codes, tr.scales, tr.biases, tr.rows, tr.cols)


def bf16_f64(bits) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def oracle_model(spec: synth.Qwen3Spec, m: dict, with_embed: bool = True) -> dict:
    layers = []
    for L in m["layers"]:
        d = {name: pack(L[name]) for name in MATS}
        d.update({name: bf16_f64(L[name]) for name in NORMS})
        layers.append(d)
    return {"hidden": spec.hidden, "heads": spec.heads, "kv_heads": spec.kv_heads,
            "head_dim": spec.head_dim, "inter": spec.inter, "vocab": spec.vocab,
            "eps": float(np.float32(spec.eps)), "theta": float(np.float32(spec.theta)),
            "layers": layers, "final_norm": bf16_f64(m["final_norm"]),
            "embed": pack(m["embed"]) if with_embed else None}


def empty_caches(spec: synth.Qwen3Spec, rows: int, layers: int):
    shape = (rows, spec.kv_heads, spec.head_dim)
    return ([np.zeros(shape) for _ in range(layers)], [np.zeros(shape) for _ in range(layers)])
