"""Pins of the decoder-step oracle (turbospark-runtime 0.3.0,
src/qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step and the kernels it
encodes: encode_rms_norm_bf16w(_perhead), encode_rope_neox_subdim,
encode_silu_mul, encode_residual_add, encode_attention_decode).

Each function is checked against something other than itself: torch's own
rms_norm and silu, hand-computed values, the algebra of rotations, an
independent numpy dequantisation, and -- for the whole step -- a plain
full-sequence (prefill) Qwen3 decoder in torch (causal mask, repeat_kv,
complex-number RoPE) whose last row must equal the cached step.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import synth
from oracle import reference_np
from qwen3_models import empty_caches, oracle_model


def test_round_f16_is_direct_nearest_even():
    v = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 1 + 2 ** -11 + 2 ** -40, 65504.0, 65519.0,
                  2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, -(1 + 2 ** -11)])
    want = np.array([1.0, 1 + 2 ** -9, 1 + 2 ** -10, 65504.0, 65504.0, 2.0 ** -24, 0.0,
                     2.0 ** -24, -1.0])
    # the third value would round to 1.0 through an f32 intermediate
    assert np.array_equal(oracle.round_f16(v), want)


def test_rms_norm_matches_torch_and_closed_form():
    g = np.random.default_rng(0)
    x = g.standard_normal((3, 256)) * 5
    w = g.normal(1.0, 0.1, 256)
    got = oracle.rms_norm(x, w, 1e-6)
    ref = F.rms_norm(torch.from_numpy(x), (256,), torch.from_numpy(w), 1e-6).numpy()
    assert np.allclose(got, ref, rtol=1e-14, atol=0)
    # a constant row c: c / sqrt(c^2 + eps) * w
    c = np.full(64, -3.0)
    assert np.allclose(oracle.rms_norm(c, np.arange(64.0), 0.25),
                       -3.0 / math.sqrt(9.25) * np.arange(64.0), rtol=1e-15)
    # per head over the last axis
    q = g.standard_normal((16, 128))
    wq = g.normal(1.0, 0.1, 128)
    for h in (0, 7, 15):
        assert np.allclose(oracle.rms_norm(q, wq, 1e-6)[h], oracle.rms_norm(q[h], wq, 1e-6))


def test_rope_neox_hand_values_and_rotation_algebra():
    x = np.array([1.0, 2.0, 3.0, 4.0])
    # d = 4, theta = 10000, position 1: angles 1 and 10000^-0.5 = 0.01
    c0, s0, c1, s1 = math.cos(1), math.sin(1), math.cos(0.01), math.sin(0.01)
    want = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 3 * c0 + 1 * s0, 4 * c1 + 2 * s1]
    assert np.allclose(oracle.rope_neox(x, 1, 10000.0), want, rtol=1e-15)
    g = np.random.default_rng(1)
    q = g.standard_normal((4, 128))
    k = g.standard_normal((4, 128))
    assert np.array_equal(oracle.rope_neox(q, 0, 1e6), q)
    # rotations compose, preserve each pair's norm, and scores depend on m - n only
    assert np.allclose(oracle.rope_neox(oracle.rope_neox(q, 17, 1e6), 25, 1e6),
                       oracle.rope_neox(q, 42, 1e6), rtol=1e-12, atol=1e-12)
    r = oracle.rope_neox(q, 1234, 1e6)
    assert np.allclose(r[:, :64] ** 2 + r[:, 64:] ** 2, q[:, :64] ** 2 + q[:, 64:] ** 2)
    s1 = np.sum(oracle.rope_neox(q, 100, 1e6) * oracle.rope_neox(k, 90, 1e6), axis=1)
    s2 = np.sum(oracle.rope_neox(q, 1010, 1e6) * oracle.rope_neox(k, 1000, 1e6), axis=1)
    assert np.allclose(s1, s2, rtol=1e-10)


def test_silu_mul_matches_torch():
    g = np.random.default_rng(2)
    a, b = g.standard_normal(1000) * 8, g.standard_normal(1000)
    ref = (F.silu(torch.from_numpy(a)) * torch.from_numpy(b)).numpy()
    assert np.allclose(oracle.silu_mul(a, b), ref, rtol=1e-14, atol=1e-300)
    assert oracle.silu_mul(np.array([0.0]), np.array([5.0]))[0] == 0.0


def test_affine_gemv_f64_matches_independent_dequant():
    tr = synth.affine_triplet(96, 320, key=(21, 0, 0), scale_range=(1e-4, 1e-3))
    blob = oracle.affine_pack(tr.codes, tr.scales, tr.biases, 96, 320)
    x = np.random.default_rng(3).standard_normal(320)
    ref = reference_np.affine_dense(blob, 96, 320) @ x
    assert np.allclose(oracle.affine_gemv_f64(blob, 96, 320, x), ref, rtol=1e-13, atol=1e-13)
    sel = np.array([95, 0, 17])
    assert np.allclose(oracle.affine_gemv_f64(blob, 96, 320, x, row_sel=sel), ref[sel],
                       rtol=1e-13, atol=1e-13)


def _prefill_reference(spec, om, X):
    """Plain full-sequence Qwen3 decoder in torch f64 (causal mask, repeat_kv,
    RoPE as a complex rotation), dense weights from the independent numpy
    dequantisation; returns the hidden rows after the last layer, the logits
    of the last row and each layer's rotated K and V rows [T, kv_heads, d]."""
    T = X.shape[0]
    hid, H, KV, d = spec.hidden, spec.heads, spec.kv_heads, spec.head_dim
    eps = om["eps"]
    scale = float(np.float32(1.0) / np.sqrt(np.float32(d)))
    dense = lambda blob, r, c: torch.from_numpy(reference_np.affine_dense(blob, r, c))
    t = torch.arange(T, dtype=torch.float64)
    inv = om["theta"] ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(T, d // 2, dtype=torch.float64), t[:, None] * inv[None, :])

    def rope(z):  # [T, heads, d]
        zc = torch.complex(z[..., :d // 2], z[..., d // 2:]) * rot[:, None, :]
        return torch.cat([zc.real, zc.imag], dim=-1)

    x = torch.from_numpy(X)
    mask = torch.triu(torch.ones(T, T, dtype=torch.bool), diagonal=1)
    kv_rows = []
    for L in om["layers"]:
        w = lambda name: torch.from_numpy(np.asarray(L[name]))
        h = F.rms_norm(x, (hid,), w("in_norm"), eps)
        q = (h @ dense(L["q"], H * d, hid).T).view(T, H, d)
        k = (h @ dense(L["k"], KV * d, hid).T).view(T, KV, d)
        v = (h @ dense(L["v"], KV * d, hid).T).view(T, KV, d)
        q = rope(F.rms_norm(q, (d,), w("q_norm"), eps))
        k = rope(F.rms_norm(k, (d,), w("k_norm"), eps))
        kv_rows.append((k.numpy().copy(), v.numpy().copy()))
        k = k.repeat_interleave(H // KV, dim=1)
        v = v.repeat_interleave(H // KV, dim=1)
        s = torch.einsum("thd,shd->hts", q, k) * scale
        p = torch.softmax(s.masked_fill(mask, float("-inf")), dim=-1)
        o = torch.einsum("hts,shd->thd", p, v).reshape(T, H * d)
        x = x + o @ dense(L["o"], hid, H * d).T
        h = F.rms_norm(x, (hid,), w("post_norm"), eps)
        a = F.silu(h @ dense(L["gate"], spec.inter, hid).T) * (h @ dense(L["up"], spec.inter, hid).T)
        x = x + a @ dense(L["down"], hid, spec.inter).T
    last = F.rms_norm(x[-1], (hid,), torch.from_numpy(om["final_norm"]), eps)
    logits = last @ dense(om["embed"], spec.vocab, hid).T
    return x.numpy(), logits.numpy(), kv_rows


def test_cached_step_equals_full_sequence_decoder():
    spec = synth.QWEN3_TINY_STEP
    om = oracle_model(spec, synth.qwen3_model(spec))
    T = 6
    X = np.random.default_rng(4).standard_normal((T, spec.hidden)) * 0.05
    ref_x, ref_logits, ref_kv = _prefill_reference(spec, om, X)
    kc, vc = empty_caches(spec, T + 2, spec.layers)
    for pos in range(T):
        x, logits = oracle.qwen3_step(X[pos], pos, om, kc, vc, f16=False)
        assert np.allclose(x, ref_x[pos], rtol=1e-11, atol=1e-11 * np.abs(ref_x[pos]).max())
    assert np.allclose(logits, ref_logits, rtol=1e-10, atol=1e-10 * np.abs(ref_logits).max())
    # the cache holds every position's rotated K and its V (absolute
    # positions: a constant shift would leave the outputs unchanged)
    for li, (rk, rv) in enumerate(ref_kv):
        assert np.allclose(kc[li][:T], rk, rtol=1e-11, atol=1e-11)
        assert np.allclose(vc[li][:T], rv, rtol=1e-11, atol=1e-11)
    # the rows past the last position were never written
    assert not kc[0][T:].any() and not vc[1][T:].any()


def test_f16_step_stores_f16_values_near_the_exact_step():
    spec = synth.QWEN3_TINY_STEP
    om = oracle_model(spec, synth.qwen3_model(spec))
    X = oracle.round_f16(np.random.default_rng(5).standard_normal((3, spec.hidden)) * 0.05)
    k16, v16 = empty_caches(spec, 4, spec.layers)
    k64, v64 = empty_caches(spec, 4, spec.layers)
    for pos in range(3):
        x16, l16 = oracle.qwen3_step(X[pos], pos, om, k16, v16, f16=True)
        x64, l64 = oracle.qwen3_step(X[pos], pos, om, k64, v64, f16=False)
    for a in (x16, l16, k16[1], v16[0]):
        assert np.array_equal(oracle.round_f16(a), a)
    # the f16 buffers move the result by rounding-sized amounts only
    assert oracle.normwise_error(x16, x64) < 2e-3
    assert oracle.normwise_error(l16, l64) < 2e-3
