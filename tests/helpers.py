"""Host <-> device marshalling and comparison helpers for the GPU tests.

Inputs come from ``synth`` (seeded), expected values from ``oracle`` only.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import quantized_transformer_decode_amd as qd

DEV = "cuda:0"

TOL_BF16 = 2e-3   # normwise bound for BF16 outputs
TOL_F32 = 1e-4    # normwise bound for f32 outputs


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).to(DEV)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).copy()).to(DEV)


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_bf16_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def pack_on_device(tr) -> torch.Tensor:
    """The affine blob built by the library's loader entry point."""
    codes = dev_u8(tr.codes)
    sc = dev_u8(tr.scales)
    bi = dev_u8(tr.biases)
    blob = torch.empty(qd.affine_i8_g64_bytes(tr.rows, tr.cols), dtype=torch.uint8, device=DEV)
    qd.affine_i8_g64_pack(codes, sc, bi, tr.rows, tr.cols, blob)
    return blob


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of BF16 numbers in the binade of |v| (normal range)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def bf16_rounding_interval(got: np.ndarray):
    """[lo, hi] of the reals that round (nearest even) to each BF16 value."""
    g = np.asarray(got, dtype=np.float64)
    u = bf16_ulp(g)
    pow2 = (g != 0) & (np.abs(g) == 2.0 ** np.floor(np.log2(np.maximum(np.abs(g), 1e-300))))
    toward0 = np.where(pow2, u / 4, u / 2)  # the binade below is twice as fine
    away = u / 2
    lo = np.where(g >= 0, g - toward0, g - away)
    hi = np.where(g >= 0, g + away, g + toward0)
    return lo, hi


def check_bf16_output(got_f64: np.ndarray, ref_f64: np.ndarray, what: str = "",
                      noise: float = 1e-5) -> float:
    """BF16 outputs (8 significant bits, unit roundoff 2^-8) cannot all lie
    within 2e-3 of the exact value even when correctly rounded, so the 2e-3
    bar applies to the kernel's value before its single BF16 store:
      * pre-rounding error -- the distance from each exact value to the set
        of reals that round to the stored output, over max |ref| -- must be
        <= 2e-3 (the stated bar) and <= `noise` (fp32 accumulation noise:
        the output is the correctly rounded exact result up to that noise);
      * the stored values themselves are within 2^-8 (+ noise) normwise.
    Returns the pre-rounding normwise error."""
    got = np.asarray(got_f64, dtype=np.float64)
    ref = np.asarray(ref_f64, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite outputs"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    lo, hi = bf16_rounding_interval(got)
    dist = np.maximum(0.0, np.maximum(lo - ref, ref - hi))
    pre = float(dist.max()) / scale if scale > 0 else float(dist.max())
    assert pre <= TOL_BF16, f"{what}: pre-rounding normwise {pre:.3e} > {TOL_BF16}"
    bad = dist > noise * scale
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs are not the rounding of " \
        f"the exact value, e.g. got {got[bad][:3]} ref {ref[bad][:3]}"
    stored = oracle.normwise_error(got, ref)
    assert stored <= 2.0 ** -8 + noise, f"{what}: stored normwise {stored:.3e}"
    return pre


def dev_f16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.float16)


def f16_rounding_interval(got: np.ndarray):
    """[lo, hi] of the reals that round (nearest even) to each f16 value
    (finite values; subnormal spacing 2^-24)."""
    g = np.asarray(got, dtype=np.float64)
    a = np.abs(g)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    u = 2.0 ** (e - 10)                                   # spacing in |g|'s binade
    pow2 = (a >= 2.0 ** -13) & (a == 2.0 ** np.floor(np.log2(np.maximum(a, 1e-300))))
    toward0 = np.where(pow2, u / 4, u / 2)                # the binade below is twice as fine
    away = u / 2
    lo = np.where(g >= 0, g - toward0, g - away)
    hi = np.where(g >= 0, g + away, g + toward0)
    return lo, hi


def check_f16_output(got_f64: np.ndarray, ref_f64: np.ndarray, what: str = "",
                     noise: float = 1e-5, allowance=None) -> float:
    """f16 outputs: as check_bf16_output with f16's rounding (11 significant
    bits): each stored value is the nearest-even rounding of the exact value
    up to `noise` (fp32 accumulation), and the stored values are within 2^-11
    (+ noise) normwise.  `allowance` (absolute, per output) widens the first
    check where a hidden f16 input of the op may round either way
    (near_tie_allowance)."""
    got = np.asarray(got_f64, dtype=np.float64)
    ref = np.asarray(ref_f64, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite outputs"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    lo, hi = f16_rounding_interval(got)
    dist = np.maximum(0.0, np.maximum(lo - ref, ref - hi))
    if allowance is not None:
        dist = np.maximum(0.0, dist - np.asarray(allowance, dtype=np.float64))
    pre = float(dist.max()) / scale if scale > 0 else float(dist.max())
    assert pre <= TOL_BF16, f"{what}: pre-rounding normwise {pre:.3e} > {TOL_BF16}"
    bad = dist > noise * scale
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs are not the rounding of " \
        f"the exact value, e.g. got {got[bad][:3]} ref {ref[bad][:3]}"
    stored = oracle.normwise_error(got, ref)
    assert stored <= 2.0 ** -11 + noise, f"{what}: stored normwise {stored:.3e}"
    return pre


def check_f32_output(got: np.ndarray, ref_f64: np.ndarray, what: str = "") -> float:
    err = oracle.normwise_error(got, ref_f64)
    assert err <= TOL_F32, f"{what}: normwise {err:.3e} > {TOL_F32}"
    return err


def near_ties(exact: np.ndarray, rel: float):
    """For values an op rounds to f16 inside a kernel (never stored): the
    nearest-even roundings r, the other neighbour alt, and where the exact
    value lies within rel * |exact| of the midpoint between them (so an fp32
    computation may land on either side)."""
    x = np.asarray(exact, dtype=np.float64)
    r = oracle.round_f16(x)
    toward = np.where(x > r, np.inf, -np.inf).astype(np.float16)
    alt = np.nextafter(r.astype(np.float16), toward).astype(np.float64)
    near = np.abs(x - (r + alt) / 2) <= rel * np.abs(x)
    return r, alt, near


def near_tie_allowance(w_cols: np.ndarray, r: np.ndarray, alt: np.ndarray,
                       near: np.ndarray) -> np.ndarray:
    """Largest change of a product W x when the near-tie entries of x take
    their other rounding: sum over those columns of |W[:, c]| |alt - r|
    (w_cols: the dense columns W[:, near])."""
    u = np.abs(alt - r)[near]
    return np.abs(w_cols) @ u if u.size else 0.0
