"""CPU checks of the comparison helpers the GPU tests rely on."""
import numpy as np
import torch

from helpers import bf16_rounding_interval, check_bf16_output


def test_rounding_interval_contains_exactly_the_preimage():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 10, [4.0, -4.0, 1.0, 0.5, 3.99, 4.01]])
    g = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).double().numpy()
    lo, hi = bf16_rounding_interval(g)
    vv = v.astype(np.float32).astype(np.float64)
    assert np.all((vv >= lo) & (vv <= hi))
    # the interval is tight: stepping just outside rounds elsewhere
    for x in (lo - 1e-6 * np.abs(lo), hi + 1e-6 * np.abs(hi)):  # beyond f32 spacing
        r = torch.from_numpy(x.astype(np.float64)).to(torch.bfloat16).double().numpy()
        assert np.all(r != g)


def test_check_accepts_correct_rounding_and_rejects_offsets():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((4, 500)) * 7
    got = torch.from_numpy(ref).float().to(torch.bfloat16).double().numpy()
    check_bf16_output(got, ref)
    bad = got.copy()
    bad[0, 3] = np.nextafter(np.float32(bad[0, 3]), np.float32(np.inf)) + abs(bad[0, 3]) * 2 ** -7
    try:
        check_bf16_output(bad, ref)
    except AssertionError:
        return
    raise AssertionError("an output one BF16 step off was accepted")


def test_f16_rounding_interval_matches_numpy():
    # every double lies in the interval of its own f16 rounding, and the next
    # double above the interval rounds elsewhere
    from helpers import f16_rounding_interval
    rng = np.random.default_rng(0)
    v = rng.standard_normal(100000) * 10.0 ** rng.integers(-7, 4, 100000)
    g = v.astype(np.float16).astype(np.float64)
    ok = np.isfinite(g)
    lo, hi = f16_rounding_interval(g[ok])
    assert np.all((v[ok] >= lo) & (v[ok] <= hi))
    assert np.all(np.nextafter(hi, np.inf).astype(np.float16).astype(np.float64) != g[ok])
    assert np.all(np.nextafter(lo, -np.inf).astype(np.float16).astype(np.float64) != g[ok])
