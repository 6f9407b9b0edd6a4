"""Pins for the oracle's Q4_0 encoder, block decode and matmul.

Page: fuel-transformers 0.19.1, src/models/lazy_quantized_whisper.rs --
module documentation (ggml Q4_0), quantize_in_out_to_q4_0 (block stream,
padding, u32 view), q_linear (matmul over the stream).

Each pin is independent of the oracle's own code: hand-derived bytes
(tests/golden), closed forms, numpy/torch library routines, exact algebraic
identities and the format's error bound.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import reference_np
import synth


def test_hand_blocks_encode(hand_blocks):
    for name, x, d, want in hand_blocks:
        got = oracle.q4_0_quantize(x, 1, 32)
        # one block = 18 bytes -> odd block count -> 2 zero pad bytes
        assert got.size == 20, name
        assert np.array_equal(got[:18], want), (name, got[:18].tobytes().hex())
        assert np.array_equal(got[18:], [0, 0]), name
        # the stored delta is f16(d) (numpy's own f16 cast)
        assert got[:2].view(np.float16)[0] == np.float16(d), name
        assert np.signbit(got[:2].view(np.float16)[0]) == np.signbit(d), name


def test_hand_block_A_decodes_to_hand_values(hand_blocks):
    # block A: d = 2, nibbles trunc((j+1)/2) except j=31 (clamped to 15)
    _, x, _, want = hand_blocks[0]
    q = np.array([min(15, (j + 1) // 2) for j in range(31)] + [15])
    expect = 2.0 * (q - 8)
    got = np.array([oracle.q4_0_weight(want, 32, 0, k) for k in range(32)])
    assert np.array_equal(got, expect)
    assert got[1] == -14.0 and got[31] == 14.0  # the tie and the clamp


def test_hand_blocks_gemv_closed_form(hand_blocks):
    # K=32, x_j = 1 -> y = sum_j d (q_j - 8) = sum of decoded weights
    _, _, _, blk = hand_blocks[0]
    x = np.ones((1, 32), dtype=np.float32)
    y = oracle.q4_0_gemm(blk, 1, 32, x)
    q = np.array([min(15, (j + 1) // 2) for j in range(31)] + [15])
    assert y[0, 0] == 2.0 * np.sum(q - 8)
    # zero block (nibbles 8) and any x -> exactly 0
    _, _, _, zb = hand_blocks[1]
    xr = np.random.default_rng(0).standard_normal((3, 32)).astype(np.float32)
    assert np.all(oracle.q4_0_gemm(zb, 1, 32, xr) == 0.0)


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 32), (2, 64), (5, 96), (4, 256)])
def test_stream_size_and_pad(rows, cols):
    w = synth.w_f32(rows, cols, key=(90, rows, cols))
    s = oracle.q4_0_quantize(w, rows, cols)
    nb = rows * cols // 32
    assert s.size == oracle.q4_0_bytes(rows, cols)
    assert s.size % 4 == 0
    if nb % 2:
        assert s.size == nb * 18 + 2 and np.all(s[-2:] == 0)
    else:
        assert s.size == nb * 18
    # the u32 word stream is the little-endian view of the bytes
    words = s.view("<u4")
    assert np.array_equal(words.view(np.uint8), s)
    assert int(words[0]) == int(s[0]) | int(s[1]) << 8 | int(s[2]) << 16 | int(s[3]) << 24


def test_block_stream_is_row_major():
    # every element of row n, block b holds 100*n + b + j/64: the block at
    # stream index n*(cols/32)+b must decode to that row's values.
    rows, cols = 3, 96
    w = np.zeros((rows, cols), dtype=np.float32)
    for n in range(rows):
        for k in range(cols):
            w[n, k] = 100 * n + k // 32 + 1 + (k % 32) / 64.0
    s = oracle.q4_0_quantize(w, rows, cols)
    for n in range(rows):
        for b in range(cols // 32):
            blk = s[18 * (n * 3 + b): 18 * (n * 3 + b) + 18]
            d = float(blk[:2].view(np.float16)[0])
            # largest element of the block is its last one (positive) -> d < 0
            assert d == pytest.approx(-(100 * n + b + 1 + 31 / 64) / 8, rel=1e-3)


def test_in_out_transpose_matches_out_in():
    # the bake receives [in, out] and transposes it to [out, in] first
    w_out_in = synth.w_f32(64, 96, key=(91, 0, 0))
    a = oracle.q4_0_quantize(w_out_in, 64, 96)
    b = oracle.q4_0_quantize_in_out(np.ascontiguousarray(w_out_in.T), 96, 64)
    assert np.array_equal(a, b)


def _decode_exact_f32(stream, rows, cols):
    return reference_np.q4_0_dense(stream, rows, cols).astype(np.float32)


def test_idempotent_requantize():
    # quantize(dequantize(B)) == B for every block: the element with q = 0
    # recreates max = -8*d exactly and the rest land within 2^-20 of k + 1/2.
    w = synth.w_f32(256, 256, key=(92, 0, 0))
    s = oracle.q4_0_quantize(w, 256, 256)
    wd = _decode_exact_f32(s, 256, 256)
    s2 = oracle.q4_0_quantize(wd, 256, 256)
    assert np.array_equal(s, s2)


def test_error_bound():
    # |x - xhat| <= |d| (1/2 + 8 * 2^-11) for unclamped elements (rounding
    # error plus the f16 rounding of d times |q-8| <= 8); <= |d| (1 + 2^-7)
    # when the nibble was clamped to 15.
    rows, cols = 128, 512
    w = synth.w_f32(rows, cols, key=(93, 0, 0))
    s = oracle.q4_0_quantize(w, rows, cols)
    dense = reference_np.q4_0_dense(s, rows, cols)
    nb = rows * cols // 32
    blk = s[: nb * 18].reshape(nb, 18)
    d = np.abs(blk[:, :2].copy().view(np.float16).astype(np.float64)).reshape(nb, 1)
    err = np.abs(w.reshape(nb, 32).astype(np.float64) - dense.reshape(nb, 32))
    hi = (blk[:, 2:] >> 4)
    clamped = np.zeros((nb, 32), dtype=bool)
    clamped[:, 16:] = hi == 15
    clamped[:, :16] = (blk[:, 2:] & 15) == 15
    lim = np.where(clamped, d * (1 + 2.0 ** -7), d * (0.5 + 8 * 2.0 ** -11))
    assert np.all(err <= lim * (1 + 1e-6))


@pytest.mark.parametrize("rows,cols", [(7, 64), (33, 128), (16, 512)])
def test_encoder_matches_numpy_restatement(rows, cols):
    w = synth.w_f32(rows, cols, key=(94, rows, cols))
    w[0, :32] = 0.0           # zero block
    w[1, 5] = 1e-7            # tiny values
    w[2, 3] = -w[2, 3:35].__abs__().max() * 1.0  # a negative maximum
    assert np.array_equal(oracle.q4_0_quantize(w, rows, cols),
                          reference_np.q4_0_quantize(w, rows, cols))


def test_gemm_all_unit_deltas_is_integer_matmul():
    # all d = 1 -> y = x (Q - 8)^T, a plain matmul (torch, f64)
    rows, cols, m = 24, 128, 5
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(rows, cols))
    nb = rows * cols // 32
    blk = np.zeros((nb, 18), dtype=np.uint8)
    blk[:, 0:2] = np.array([np.float16(1.0)]).view(np.uint8)
    qb = q.reshape(nb, 32)
    blk[:, 2:] = (qb[:, :16] | (qb[:, 16:] << 4)).astype(np.uint8)
    stream = blk.reshape(-1)
    x = rng.standard_normal((m, cols)).astype(np.float32)
    y = oracle.q4_0_gemm(stream, rows, cols, x)
    ref = torch.from_numpy(x.astype(np.float64)) @ torch.from_numpy((q - 8).astype(np.float64)).T
    assert np.allclose(y, ref.numpy(), rtol=0, atol=1e-12 * np.abs(ref.numpy()).max())


def test_gemm_one_hot_reads_single_weight():
    rows, cols = 6, 64
    w = synth.w_f32(rows, cols, key=(95, 0, 0))
    s = oracle.q4_0_quantize(w, rows, cols)
    blk = s[: rows * cols // 32 * 18].reshape(-1, 18)
    x = np.eye(cols, dtype=np.float32)
    y = oracle.q4_0_gemm(s, rows, cols, x)  # [cols, rows]
    for n in range(rows):
        for k in range(cols):
            b = blk[n * 2 + k // 32]
            d = float(b[:2].view(np.float16)[0])
            j = k % 32
            q = (b[2 + j] & 15) if j < 16 else (b[2 + j - 16] >> 4)
            assert y[k, n] == d * (int(q) - 8)


def test_gemm_bf16_input_and_scaling():
    rows, cols, m = 16, 256, 3
    s = oracle.q4_0_quantize(synth.w_f32(rows, cols, key=(96, 0, 0)), rows, cols)
    xb = synth.x_bf16(m, cols, key=(96, 0, 1))
    xf = synth.bf16_bits_to_f32(xb)
    assert np.array_equal(oracle.q4_0_gemm(s, rows, cols, xb),
                          oracle.q4_0_gemm(s, rows, cols, xf))
    # y(2x) == 2 y(x) exactly (doubling is exact in f32 and f64)
    assert np.array_equal(oracle.q4_0_gemm(s, rows, cols, 2 * xf),
                          2 * oracle.q4_0_gemm(s, rows, cols, xf))


def test_gemm_matches_numpy_and_selection():
    rows, cols, m = 40, 320, 4
    s = oracle.q4_0_quantize(synth.w_f32(rows, cols, key=(97, 0, 0)), rows, cols)
    x = synth.x_f32(m, cols, key=(97, 0, 1))
    y = oracle.q4_0_gemm(s, rows, cols, x)
    ref = x.astype(np.float64) @ reference_np.q4_0_dense(s, rows, cols).T
    assert oracle.normwise_error(y, ref) < 1e-12
    ys = oracle.q4_0_gemm(s, rows, cols, x, m_sel=[3, 0], row_sel=[39, 7, 7])
    assert np.array_equal(ys, y[[3, 0]][:, [39, 7, 7]])


# ---- q_linear: bias and gelu_tanh -------------------------------------------

def test_gelu_tanh_matches_torch_and_known_values():
    # torch's tanh-approximate GELU (an independent implementation) in f64,
    # and values fixed by the formula: gelu(0) = 0, gelu(1) = 0.84119199...,
    # gelu(v) -> v for large v, -> 0 for very negative v
    v = np.concatenate([np.linspace(-12, 12, 2001), [0.0, 1.0, -1.0, 40.0, -40.0]])
    want = torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    got = oracle.gelu_tanh(v)
    assert np.max(np.abs(got - want)) <= 1e-15 * np.max(np.abs(want))
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert abs(oracle.gelu_tanh(np.array([1.0]))[0] - 0.8411919906082768) < 1e-15
    assert oracle.gelu_tanh(np.array([40.0]))[0] == 40.0
    assert abs(oracle.gelu_tanh(np.array([-40.0]))[0]) < 1e-300


def test_q_linear_bias_closed_form():
    # all-zero weights (d = 0): the output is the bias, broadcast over tokens
    rows, cols, m = 48, 256, 5
    wq = oracle.q4_0_quantize(np.zeros((rows, cols), np.float32), rows, cols)
    bias = synth.w_f32(1, rows, std=1.0, key=(84, 0, 0)).reshape(-1)
    x = synth.x_f32(m, cols, key=(84, 0, 1))
    y = oracle.q_linear(wq, rows, cols, x, bias)
    assert np.array_equal(y, np.broadcast_to(bias.astype(np.float64), (m, rows)))
    g = oracle.q_linear(wq, rows, cols, x, bias, gelu=True)
    assert np.array_equal(g, oracle.gelu_tanh(np.broadcast_to(bias.astype(np.float64), (m, rows))))


def test_q_linear_is_gemm_plus_bias_on_selections():
    rows, cols, m = 40, 512, 6
    wq = oracle.q4_0_quantize(synth.w_f32(rows, cols, key=(85, 0, 0)), rows, cols)
    x = synth.x_f32(m, cols, key=(85, 0, 1))
    bias = synth.w_f32(1, rows, std=0.5, key=(85, 0, 2)).reshape(-1)
    full = oracle.q_linear(wq, rows, cols, x, bias, gelu=True)
    part = oracle.q_linear(wq, rows, cols, x, bias, gelu=True, m_sel=[5, 0], row_sel=[39, 2, 7])
    assert np.array_equal(part, full[np.ix_([5, 0], [39, 2, 7])])
    plain = oracle.q4_0_gemm(wq, rows, cols, x)
    assert np.array_equal(oracle.q_linear(wq, rows, cols, x), plain)
