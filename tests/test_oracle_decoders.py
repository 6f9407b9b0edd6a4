"""Pins for the oracle's IEEE half / bfloat16 decoders and its f32 -> f16
round-to-nearest-even encoder, against numpy's and torch's own casts
(library routines that implement the same IEEE definitions)."""
import numpy as np
import pytest
import torch

import oracle


def _all_bits():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_f16_decoder_all_bit_patterns():
    bits = _all_bits()
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # the sign of zero is kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_bf16_decoder_all_bit_patterns():
    bits = _all_bits()
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _edge_f32():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e30,
            -1e30, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -26,
            5 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
            2.0 ** -14 - 2.0 ** -26, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11,
            1.0 + 2.0 ** -11 + 2.0 ** -23, 2047.5, 2048.5, 4095.0,
            float("inf"), float("-inf"), 1e-40, -1e-45, 0.1, 1 / 3]
    out = []
    for v in vals:
        f = np.float32(v)
        out.extend([f, -f, np.nextafter(f, np.float32(np.inf)),
                    np.nextafter(f, np.float32(-np.inf))])
    return np.array(out, dtype=np.float32)


def test_f32_to_f16_rne_edges():
    x = _edge_f32()
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_rne(v) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref), [(float(a), hex(b), hex(c)) for a, b, c in
                                      zip(x, got, ref) if b != c]


@pytest.mark.parametrize("seed", [0, 1])
def test_f32_to_f16_rne_random(seed):
    rng = np.random.default_rng(seed)
    # random bit patterns over the whole f32 exponent range near f16's
    e = rng.integers(127 - 30, 127 + 18, size=20000).astype(np.uint32)
    m = rng.integers(0, 1 << 23, size=20000).astype(np.uint32)
    s = rng.integers(0, 2, size=20000).astype(np.uint32)
    x = ((s << 31) | (e << 23) | m).view(np.float32)
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_rne(v) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_f32_to_f16_nan_is_nan():
    h = oracle.f32_to_f16_rne(float("nan"))
    assert np.isnan(np.uint16(h).view(np.float16))
