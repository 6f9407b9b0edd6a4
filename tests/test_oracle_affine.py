"""Pins for the oracle's affine-INT8 g64 layout, dequant and GEMV.

Page: turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs --
PackedLinear::resident (offsets), load_packed_linear (blob order and byte
counts), embed_row_bytes (w = q as f32 * scale + bias, group
row*groups + col/64, little-endian BF16).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import reference_np
import synth


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).float().numpy()


def _blob(tr):
    return oracle.affine_pack(tr.codes, tr.scales, tr.biases, tr.rows, tr.cols)


@pytest.mark.parametrize("rows,cols,so,bo,total", [
    (1024, 1024, 1048576, 1048576 + 32768, 1114112),
    (151936, 1024, 155582464, 155582464 + 4861952, 155582464 + 2 * 4861952),
    (2, 64, 128, 132, 136),
])
def test_offsets_page_formula(rows, cols, so, bo, total):
    # weights at 0; scales at rows*cols; biases at rows*cols + rows*(cols/64)*2
    assert oracle.affine_scales_offset(rows, cols) == so == rows * cols
    assert oracle.affine_biases_offset(rows, cols) == bo
    assert oracle.affine_bytes(rows, cols) == total


def test_pack_is_concatenation():
    tr = synth.affine_triplet(48, 192, key=(80, 0, 0))
    blob = _blob(tr)
    want = np.concatenate([tr.codes.view(np.uint8).reshape(-1),
                           tr.scales.view(np.uint8).reshape(-1),
                           tr.biases.view(np.uint8).reshape(-1)])
    assert np.array_equal(blob, want)
    # code (r, c) is byte r*cols + c of the little-endian u32 words
    w = tr.codes
    r, c = 5, 77
    word = int(w[r, c // 4])
    assert blob[r * 192 + c] == (word >> (8 * (c % 4))) & 0xFF


def test_brute_force_k64_closed_form():
    # q_c = c, x_c = 1, s = 2^-8, b = -0.5 -> y = 2016/256 - 32 = -24.125
    codes = np.arange(64, dtype=np.uint8).reshape(1, 64)
    tr = synth.affine_triplet_custom(codes, np.array([[2.0 ** -8]]), np.array([[-0.5]]))
    x = synth.to_bf16_bits(np.ones((1, 64), dtype=np.float32))
    y = oracle.affine_gemv(_blob(tr), 1, 64, x)
    assert y[0, 0] == -24.125


def test_one_hot_equals_page_f32_formula():
    # x = e_c -> y[r] = w[r, c]; the page computes q as f32 * scale + bias in
    # f32, which is exact here (q*scale has <= 16 significant bits), so the
    # f64 oracle must round to exactly that f32 value.
    rows, cols = 8, 192
    tr = synth.affine_triplet(rows, cols, key=(81, 0, 0))
    blob = _blob(tr)
    eye = synth.to_bf16_bits(np.eye(cols, dtype=np.float32))
    y = oracle.affine_gemv(blob, rows, cols, eye)  # [cols, rows]
    q = tr.codes.view(np.uint8).reshape(rows, cols).astype(np.float32)
    s = _bf16(tr.scales)
    b = _bf16(tr.biases)
    for r in range(rows):
        for c in range(cols):
            g = c // 64
            page = np.float32(q[r, c] * s[r, g]) + b[r, g]
            assert np.float32(y[c, r]) == page, (r, c)


def test_zero_scale_gives_bias_row_sums():
    rows, cols, m = 6, 256, 3
    tr = synth.affine_triplet(rows, cols, key=(82, 0, 0))
    tr.scales[:] = 0
    x = synth.x_bf16(m, cols, key=(82, 0, 1))
    y = oracle.affine_gemv(_blob(tr), rows, cols, x)
    xf = _bf16(x).astype(np.float64).reshape(m, cols // 64, 64).sum(axis=2)  # X[m, g]
    want = xf @ _bf16(tr.biases).astype(np.float64).T
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13)


def test_constant_code_closed_form():
    rows, cols, m, q0 = 5, 320, 2, 200
    tr = synth.affine_triplet(rows, cols, key=(83, 0, 0))
    tr.codes[:] = np.uint32(q0 * 0x01010101)
    x = synth.x_bf16(m, cols, key=(83, 0, 1))
    y = oracle.affine_gemv(_blob(tr), rows, cols, x)
    X = _bf16(x).astype(np.float64).reshape(m, cols // 64, 64).sum(axis=2)
    wg = _bf16(tr.scales).astype(np.float64) * q0 + _bf16(tr.biases).astype(np.float64)
    assert np.allclose(y, X @ wg.T, rtol=1e-13, atol=1e-12)


def test_unit_scale_zero_bias_is_integer_matmul():
    rows, cols, m = 12, 128, 4
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(rows, cols)).astype(np.uint8)
    tr = synth.affine_triplet_custom(codes, np.ones((rows, 2)), np.zeros((rows, 2)))
    x = synth.x_bf16(m, cols, key=(84, 0, 0))
    y = oracle.affine_gemv(_blob(tr), rows, cols, x)
    ref = torch.from_numpy(_bf16(x).astype(np.float64)) @ torch.from_numpy(
        codes.astype(np.float64)).T
    assert np.array_equal(y, ref.numpy())  # all partial sums exact in f64


def test_group_index_per_row_and_group():
    # distinct scale per (row, group): a wrong group index changes the result
    rows, cols = 3, 256
    codes = np.full((rows, cols), 1, dtype=np.uint8)
    sc = np.array([[2.0 ** (-(r * 4 + g)) for g in range(4)] for r in range(rows)])
    tr = synth.affine_triplet_custom(codes, sc, np.zeros((rows, 4)))
    blob = _blob(tr)
    for r in range(rows):
        for c in (0, 63, 64, 130, 255):
            assert oracle.affine_weight(blob, rows, cols, r, c) == sc[r, c // 64]


def test_scaling_rows_and_selection():
    rows, cols, m = 40, 384, 5
    tr = synth.affine_triplet(rows, cols, key=(85, 0, 0))
    blob = _blob(tr)
    x = synth.x_bf16(m, cols, key=(85, 0, 1))
    y = oracle.affine_gemv(blob, rows, cols, x)
    x2 = synth.to_bf16_bits(2 * _bf16(x))
    assert np.array_equal(oracle.affine_gemv(blob, rows, cols, x2), 2 * y)
    # multi-row layout: row t of y is the GEMV of row t of x alone
    for t in range(m):
        assert np.array_equal(oracle.affine_gemv(blob, rows, cols, x[t:t + 1]), y[t:t + 1])
    ys = oracle.affine_gemv(blob, rows, cols, x, m_sel=[4, 1], row_sel=[0, 39, 17])
    assert np.array_equal(ys, y[[4, 1]][:, [0, 39, 17]])


def test_matches_numpy_restatement():
    rows, cols, m = 64, 512, 3
    tr = synth.affine_triplet(rows, cols, key=(86, 0, 0))
    blob = _blob(tr)
    x = synth.x_bf16(m, cols, key=(86, 0, 1))
    y = oracle.affine_gemv(blob, rows, cols, x)
    ref = reference_np.bf16_bits_to_f64(x) @ reference_np.affine_dense(blob, rows, cols).T
    assert oracle.normwise_error(y, ref) < 1e-13


# ---- f16 activations and the tied-embedding row ---------------------------

def _f16_bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def test_brute_force_k64_f16_input():
    # the same exact case with x given as f16 ones (0x3C00)
    codes = np.arange(64, dtype=np.uint8).reshape(1, 64)
    tr = synth.affine_triplet_custom(codes, np.array([[2.0 ** -8]]), np.array([[-0.5]]))
    x = np.full((1, 64), 0x3C00, dtype=np.uint16)
    assert oracle.affine_gemv(_blob(tr), 1, 64, x, x_f16=True)[0, 0] == -24.125


def test_gemv_f16_input_decodes_like_numpy():
    # f16 x decoded by the oracle equals numpy's float16 values (normal,
    # subnormal and signed zero inputs), through a one-hot weight row
    rows, cols = 1, 64
    codes = np.zeros((rows, cols), dtype=np.uint8)
    vals = np.array([1.5, -2.0 ** -20, 65504.0, -0.0, 2.0 ** -24, 0.333], dtype=np.float16)
    for k, v in enumerate(vals):
        codes[:] = 0
        codes[0, k] = 1
        tr = synth.affine_triplet_custom(codes, np.array([[1.0]]), np.array([[0.0]]))
        x = np.zeros((1, cols), dtype=np.uint16)
        x[0, k] = vals.view(np.uint16)[k]
        assert oracle.affine_gemv(_blob(tr), rows, cols, x, x_f16=True)[0, 0] == float(v)


def test_embed_row_double_rounding_pin():
    # embed_row_bytes rounds q*scale + bias to f32 first, then to f16.
    # q = 226, scale = 145 * 2^-26 (BF16 0x3611), bias = 1.0: the exact value
    # 1 + 2^-11 + 2^-25 becomes the f16 midpoint 1 + 2^-11 in f32, which ties
    # to even (0x3C00); rounding the exact value straight to f16 would give
    # 0x3C01.  In BF16 (ulp 2^-7 at 1) both readings give 1.0 (0x3F80).
    cols = 64
    codes = np.full((1, cols), 226, dtype=np.uint8)
    tr = synth.affine_triplet_custom(codes, np.array([[145 * 2.0 ** -26]]), np.array([[1.0]]))
    assert int(tr.scales[0, 0]) == 0x3611 and int(tr.biases[0, 0]) == 0x3F80
    blob = _blob(tr)
    assert np.all(oracle.affine_embed_row(blob, 1, cols, 0, out_f16=True) == 0x3C00)
    assert np.all(oracle.affine_embed_row(blob, 1, cols, 0, out_f16=False) == 0x3F80)


def test_embed_row_closed_forms():
    # q = 0 -> the bias itself; q = 255, s = 2^-8, b = -0.5 -> 127/256 (0x37F0)
    cols = 128
    codes = np.zeros((2, cols), dtype=np.uint8)
    codes[1, :] = 255
    sc = np.array([[1e-3, 5e-3], [2.0 ** -8, 2.0 ** -8]])
    bi = np.array([[-0.5, 0.25], [-0.5, -0.5]])
    blob = _blob(synth.affine_triplet_custom(codes, sc, bi))
    r0 = oracle.affine_embed_row(blob, 2, cols, 0)
    assert np.all(r0[:64] == 0xB800) and np.all(r0[64:] == 0x3400)
    assert np.all(oracle.affine_embed_row(blob, 2, cols, 1) == 0x37F0)
    assert np.all(oracle.affine_embed_row(blob, 2, cols, 1, out_f16=False) == 0x3EFE)


def test_embed_row_matches_numpy_f32_arithmetic():
    # numpy's float32 arithmetic and float16 / torch's bfloat16 conversions
    # (independent implementations) agree with the oracle bit for bit
    rows, cols = 40, 256
    tr = synth.affine_triplet(rows, cols, key=(81, 0, 0))
    blob = _blob(tr)
    q = tr.codes.view(np.uint8).reshape(rows, cols).astype(np.float32)
    s = np.repeat(_bf16(tr.scales), 64, axis=1).astype(np.float32)
    b = np.repeat(_bf16(tr.biases), 64, axis=1).astype(np.float32)
    v = q * s + b  # float32 product, then float32 sum
    want16 = v.astype(np.float16).view(np.uint16)
    wantb = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for r in (0, 1, 17, rows - 1):
        assert np.array_equal(oracle.affine_embed_row(blob, rows, cols, r), want16[r])
        assert np.array_equal(oracle.affine_embed_row(blob, rows, cols, r, out_f16=False),
                              wantb[r])


def test_bf16_encoder_matches_torch():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 4000),
                           np.array([0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                                     3.3895314e38, np.inf, -np.inf, 1e-40], dtype=np.float32)])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16_rne(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)
