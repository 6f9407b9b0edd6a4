"""GPU parity of the Q4_0 bake, GEMV and prefill GEMM against the oracle.

fuel-transformers 0.19.1, src/models/lazy_quantized_whisper.rs -- module
documentation and quantize_in_out_to_q4_0 (bake), q_linear (matmul),
forward_encoder / encoder_layer (prefill over all frames).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_transformer_decode_amd as qd
import synth
from conftest import load_hand_blocks
from helpers import DEV, check_f32_output, dev_bf16, dev_f32, dev_u8

pytestmark = pytest.mark.gpu


def _quantize_dev(w_host, rows, cols):
    w = dev_f32(w_host)
    out = torch.full((qd.q4_0_bytes(rows, cols),), 0xAB, dtype=torch.uint8, device=DEV)
    qd.q4_0_quantize(w, rows, cols, out)
    torch.cuda.synchronize()
    return out


def test_quantize_hand_blocks():
    blocks = load_hand_blocks()
    w = np.stack([x for _, x, _, _ in blocks]).astype(np.float32)  # 4 blocks
    got = _quantize_dev(w, 4, 32).cpu().numpy()
    for i, (name, _, _, want) in enumerate(blocks):
        assert np.array_equal(got[18 * i: 18 * i + 18], want), name
    for i, (name, x, _, want) in enumerate(blocks):
        one = _quantize_dev(x.reshape(1, 32), 1, 32).cpu().numpy()
        assert np.array_equal(one[:18], want) and np.array_equal(one[18:], [0, 0]), name


@pytest.mark.parametrize("rows,cols", [
    (2048, 512), (512, 2048),                       # Whisper-base FFN pair
    (1280, 1280), (5120, 1280), (1280, 5120),       # Whisper-large layer
    (1, 32), (3, 32), (7, 96), (13, 416), (5, 8192),  # odd counts, ragged waves
])
def test_quantize_bit_exact_random(rows, cols):
    print(f"quantize rows={rows} cols={cols}", flush=True)
    w = synth.w_f32(rows, cols, key=(2, rows, cols))
    got = _quantize_dev(w, rows, cols).cpu().numpy()
    assert np.array_equal(got, oracle.q4_0_quantize(w, rows, cols))


def test_quantize_special_values():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[0, :32] = 0.0                                  # all-zero block -> d = -0.0
    w[1, :32] = -0.0
    w[2, 5], w[2, 9] = 0.5, -0.5                     # tie on |max|: first wins
    w[3, :32] = np.float32(1e-42)                    # subnormal inputs
    w[3, 7] = np.float32(-3e-41)
    w[4, :32] = np.arange(32, dtype=np.float32) - 16  # exact ties k + 1/2
    w[5, 32:64] = 7.0                                 # constant block
    w[6, :32] = np.float32(60000.0)                   # large but in range
    w[7, :32] = rng.standard_normal(32).astype(np.float32) * 1e-30
    got = _quantize_dev(w, 64, 256).cpu().numpy()
    assert np.array_equal(got, oracle.q4_0_quantize(w, 64, 256))


@pytest.mark.parametrize("rows,cols,m", [
    (2048, 512, 1), (512, 2048, 1), (2048, 512, 4), (512, 2048, 4),
    (1280, 1280, 1), (5120, 1280, 1), (1280, 5120, 1), (1280, 5120, 4),
    (1, 256, 1), (9, 256, 3), (100, 768, 16), (37, 2816, 5),
    # the widest input the GEMV takes (8192 columns)
    (97, 8192, 4), (33, 8192, 16),
])
def test_gemv_parity(rows, cols, m):
    print(f"q4_0 gemv rows={rows} cols={cols} m={m}", flush=True)
    w = synth.w_f32(rows, cols, key=(2, rows, cols))
    wq = oracle.q4_0_quantize(w, rows, cols)
    x = synth.x_f32(m, cols, key=(2, rows, cols + m))
    y = torch.full((m, rows), float("nan"), device=DEV)
    qd.qgemv_q4_0(dev_u8(wq), rows, cols, dev_f32(x), y, m)
    torch.cuda.synchronize()
    ref = oracle.q4_0_gemm(wq, rows, cols, x)
    check_f32_output(y.cpu().numpy(), ref, f"{rows}x{cols} m={m}")


# Same-input Q4_0 groups in one launch: a Whisper decoder layer's q/k/v,
# ragged rows, tokens 1..16, and a group long enough for the streaming walk
# to cross matrix boundaries (sampled rows).
GROUPS = [((1280, 1280, 1280), 1280, 1), ((512, 512), 2048, 4), ((5, 130, 64, 9), 256, 2),
          ((300, 77), 512, 16), ((20000, 30000), 1280, 1)]


@pytest.mark.parametrize("rows_list,cols,m", GROUPS)
def test_gemv_group_parity(rows_list, cols, m):
    print(f"q4_0 gemv group rows={rows_list} cols={cols} m={m}", flush=True)
    wqs = [oracle.q4_0_quantize(synth.w_f32(r, cols, key=(8, k, r)), r, cols)
           for k, r in enumerate(rows_list)]
    x = synth.x_f32(m, cols, key=(8, cols, m))
    ws = [dev_u8(wq) for wq in wqs]
    ys = [torch.full((m, r), float("nan"), device=DEV) for r in rows_list]
    qd.qgemv_q4_0_group([(w, y, r) for w, y, r in zip(ws, ys, rows_list)], cols, dev_f32(x), m)
    torch.cuda.synchronize()
    for k, (r, wq, y) in enumerate(zip(rows_list, wqs, ys)):
        got = y.cpu().numpy()
        if r > 4096:
            sel = np.unique(np.concatenate([np.random.default_rng(k).integers(0, r, 512),
                                            np.arange(16), np.arange(r - 24, r)]))
            ref = oracle.q4_0_gemm(wq, r, cols, x, row_sel=sel)
            check_f32_output(got[:, sel], ref, f"group item {k} ({r}x{cols}) sampled")
        else:
            ref = oracle.q4_0_gemm(wq, r, cols, x)
            check_f32_output(got, ref, f"group item {k} ({r}x{cols})")


def test_gemv_zero_blocks_exact():
    # nibbles 8 (or d = 0) contribute exactly 0
    rows, cols = 64, 512
    wq = oracle.q4_0_quantize(np.zeros((rows, cols), np.float32), rows, cols)
    x = synth.x_f32(2, cols, key=(2, 0, 9))
    y = torch.full((2, rows), float("nan"), device=DEV)
    qd.qgemv_q4_0(dev_u8(wq), rows, cols, dev_f32(x), y, 2)
    torch.cuda.synchronize()
    assert np.all(y.cpu().numpy() == 0.0)


def _gemm(wq, rows, cols, x_bits, m):
    y = torch.full((m, rows), float("nan"), device=DEV)
    qd.qgemm_q4_0_prefill(dev_u8(wq), rows, cols, dev_bf16(x_bits), y, m)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("rows,cols,m", [
    (64, 256, 1), (80, 512, 15), (130, 768, 17), (320, 512, 130), (1, 256, 64),
    (1280, 1280, 65),
    # long K: the widest input the GEMM takes (65536 columns), and 16384
    (96, 65536, 3), (70, 16384, 130),
])
def test_gemm_parity_full(rows, cols, m):
    print(f"q4_0 gemm rows={rows} cols={cols} m={m}", flush=True)
    w = synth.w_f32(rows, cols, key=(5, rows, cols))
    wq = oracle.q4_0_quantize(w, rows, cols)
    x = synth.x_bf16(m, cols, key=(5, rows, cols + m))
    y = _gemm(wq, rows, cols, x, m)
    check_f32_output(y, oracle.q4_0_gemm(wq, rows, cols, x), f"{rows}x{cols} m={m}")


@pytest.mark.parametrize("rows,cols", [(1280, 1280), (5120, 1280), (1280, 5120)])
def test_gemm_whisper_large_1500_sampled(rows, cols):
    # the full encoder size (1500 frames), checked on sampled outputs
    print(f"q4_0 gemm 1500 rows={rows} cols={cols}", flush=True)
    m = 1500
    w = synth.w_f32(rows, cols, key=(5, 0, rows + cols))
    wq = oracle.q4_0_quantize(w, rows, cols)
    x = synth.x_bf16(m, cols, key=(5, 1, rows + cols))
    y = _gemm(wq, rows, cols, x, m)
    rng = np.random.default_rng(rows + cols)
    ms = np.unique(np.concatenate([rng.integers(0, m, 48), [0, 63, 64, 127, 128, 1407, 1408, 1499]]))
    rs = np.unique(np.concatenate([rng.integers(0, rows, 192), [0, 63, 64, 127, 128, rows - 1]]))
    ref = oracle.q4_0_gemm(wq, rows, cols, x, m_sel=ms, row_sel=rs)
    check_f32_output(y[np.ix_(ms, rs)], ref, f"1500x{rows}x{cols}")
    assert np.isfinite(y).all()


def test_gemm_wide_tiles_ragged_sampled():
    # enough 128 x 128 tiles for the wide kernel (40 x 12 on 256 CUs), with
    # a ragged last tile in both frames (1499) and weight rows (5000)
    rows, cols, m = 5000, 1280, 1499
    print(f"q4_0 gemm wide rows={rows} cols={cols} m={m}", flush=True)
    w = synth.w_f32(rows, cols, key=(5, 2, rows))
    wq = oracle.q4_0_quantize(w, rows, cols)
    x = synth.x_bf16(m, cols, key=(5, 3, m))
    y = _gemm(wq, rows, cols, x, m)
    rng = np.random.default_rng(rows)
    ms = np.unique(np.concatenate([rng.integers(0, m, 40),
                                   [0, 63, 64, 127, 128, 1407, 1408, 1471, 1472, m - 1]]))
    rs = np.unique(np.concatenate([rng.integers(0, rows, 160),
                                   [0, 63, 64, 127, 128, 4991, 4992, 4993, rows - 1]]))
    ref = oracle.q4_0_gemm(wq, rows, cols, x, m_sel=ms, row_sel=rs)
    check_f32_output(y[np.ix_(ms, rs)], ref, f"{m}x{rows}x{cols}")
    assert np.isfinite(y).all()


def test_gemm_rows_match_gemv():
    # each GEMM row equals the GEMV of that token (the same sum, f32 inputs
    # widened from BF16)
    rows, cols, m = 256, 1280, 20
    wq = oracle.q4_0_quantize(synth.w_f32(rows, cols, key=(6, 0, 0)), rows, cols)
    xb = synth.x_bf16(m, cols, key=(6, 0, 1))
    yg = _gemm(wq, rows, cols, xb, m)
    xf = synth.bf16_bits_to_f32(xb)
    yv = torch.empty((m, rows), device=DEV)
    for t0 in range(0, m, 16):
        mm = min(16, m - t0)
        qd.qgemv_q4_0(dev_u8(wq), rows, cols, dev_f32(xf[t0:t0 + mm]), yv[t0:t0 + mm], mm)
    torch.cuda.synchronize()
    assert oracle.normwise_error(yg, yv.cpu().numpy().astype(np.float64)) < 1e-5


# ---- q_linear: bias and gelu_tanh in the epilogue, grouped products --------

def _bias(rows, key):
    return synth.w_f32(1, rows, std=0.5, key=(11, rows, key)).reshape(-1)


@pytest.mark.parametrize("shapes,cols,m,gelu", [
    ((1280, 1280, 1280), 1280, 1, False),   # a decoder layer's q, k, v (k without bias)
    ((5120,), 1280, 1, True),               # fc1 + gelu_tanh
    ((1280,), 5120, 4, False),              # fc2
    ((33, 300), 512, 16, True),             # ragged rows, 16 tokens
])
def test_qlinear_gemv_parity(shapes, cols, m, gelu):
    print(f"qlinear gemv {shapes} cols={cols} m={m} gelu={gelu}", flush=True)
    wqs = [oracle.q4_0_quantize(synth.w_f32(r, cols, key=(12, k, r)), r, cols)
           for k, r in enumerate(shapes)]
    biases = [None if k == 1 else _bias(r, k) for k, r in enumerate(shapes)]
    x = synth.x_f32(m, cols, key=(12, cols, m))
    ys = [torch.full((m, r), float("nan"), device=DEV) for r in shapes]
    qd.qlinear_q4_0_gemv([(dev_u8(wq), None if b is None else dev_f32(b), y, r)
                          for wq, b, y, r in zip(wqs, biases, ys, shapes)],
                         cols, dev_f32(x), m, gelu=gelu)
    torch.cuda.synchronize()
    for k, (wq, b, y, r) in enumerate(zip(wqs, biases, ys, shapes)):
        ref = oracle.q_linear(wq, r, cols, x, b, gelu=gelu)
        check_f32_output(y.cpu().numpy(), ref, f"item {k} ({r}x{cols})")


@pytest.mark.parametrize("shapes,cols,m,gelu", [
    ((80, 130, 64), 512, 70, False),
    ((320,), 768, 130, True),
])
def test_qlinear_gemm_parity_full(shapes, cols, m, gelu):
    print(f"qlinear gemm {shapes} cols={cols} m={m} gelu={gelu}", flush=True)
    wqs = [oracle.q4_0_quantize(synth.w_f32(r, cols, key=(13, k, r)), r, cols)
           for k, r in enumerate(shapes)]
    biases = [None if k == 1 else _bias(r, 10 + k) for k, r in enumerate(shapes)]
    x = synth.x_bf16(m, cols, key=(13, cols, m))
    ys = [torch.full((m, r), float("nan"), device=DEV) for r in shapes]
    qd.qlinear_q4_0_gemm([(dev_u8(wq), None if b is None else dev_f32(b), y, r)
                          for wq, b, y, r in zip(wqs, biases, ys, shapes)],
                         cols, dev_bf16(x), m, gelu=gelu)
    torch.cuda.synchronize()
    for k, (wq, b, y, r) in enumerate(zip(wqs, biases, ys, shapes)):
        check_f32_output(y.cpu().numpy(), oracle.q_linear(wq, r, cols, x, b, gelu=gelu),
                         f"item {k} ({r}x{cols})")


def test_qlinear_gemm_wide_group_sampled():
    # two products sharing x with enough wide tiles (20 + 20 column tiles x
    # 12 frame tiles), biases and gelu_tanh, the second product ragged
    shapes, cols, m = (2560, 2500), 512, 1500
    print(f"qlinear gemm wide {shapes} cols={cols} m={m}", flush=True)
    wqs = [oracle.q4_0_quantize(synth.w_f32(r, cols, key=(15, k, r)), r, cols)
           for k, r in enumerate(shapes)]
    biases = [_bias(r, 30 + k) for k, r in enumerate(shapes)]
    x = synth.x_bf16(m, cols, key=(15, cols, m))
    ys = [torch.full((m, r), float("nan"), device=DEV) for r in shapes]
    qd.qlinear_q4_0_gemm([(dev_u8(wq), dev_f32(b), y, r)
                          for wq, b, y, r in zip(wqs, biases, ys, shapes)],
                         cols, dev_bf16(x), m, gelu=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(15)
    ms = np.unique(np.concatenate([rng.integers(0, m, 32), [0, 127, 128, 1407, 1408, m - 1]]))
    for k, (wq, b, y, r) in enumerate(zip(wqs, biases, ys, shapes)):
        rs = np.unique(np.concatenate([rng.integers(0, r, 96), [0, 127, 128, r - 1]]))
        got = y.cpu().numpy()
        assert np.isfinite(got).all()
        ref = oracle.q_linear(wq, r, cols, x, b, gelu=True, m_sel=ms, row_sel=rs)
        check_f32_output(got[np.ix_(ms, rs)], ref, f"item {k} ({r}x{cols})")


def test_qlinear_gemm_whisper_qkv_and_fc1_1500_sampled():
    # the encoder's fused q/k/v (3 x 1280 columns, k without bias) and fc1 +
    # gelu_tanh at 1500 frames, checked on sampled outputs
    m, d = 1500, 1280
    x = synth.x_bf16(m, d, key=(14, 0, 0))
    for shapes, gelu in (((d, d, d), False), ((5120,), True)):
        print(f"qlinear gemm 1500 {shapes} gelu={gelu}", flush=True)
        wqs = [oracle.q4_0_quantize(synth.w_f32(r, d, key=(14, k, r)), r, d)
               for k, r in enumerate(shapes)]
        biases = [None if (k == 1 and len(shapes) == 3) else _bias(r, 20 + k)
                  for k, r in enumerate(shapes)]
        ys = [torch.full((m, r), float("nan"), device=DEV) for r in shapes]
        qd.qlinear_q4_0_gemm([(dev_u8(wq), None if b is None else dev_f32(b), y, r)
                              for wq, b, y, r in zip(wqs, biases, ys, shapes)],
                             d, dev_bf16(x), m, gelu=gelu)
        torch.cuda.synchronize()
        rng = np.random.default_rng(len(shapes))
        ms = np.unique(np.concatenate([rng.integers(0, m, 32), [0, 63, 64, 1499]]))
        for k, (wq, b, y, r) in enumerate(zip(wqs, biases, ys, shapes)):
            rs = np.unique(np.concatenate([rng.integers(0, r, 96), [0, 63, 64, r - 1]]))
            got = y.cpu().numpy()
            ref = oracle.q_linear(wq, r, d, x, b, gelu=gelu, m_sel=ms, row_sel=rs)
            check_f32_output(got[np.ix_(ms, rs)], ref, f"item {k} ({r}x{d}) sampled")
            assert np.isfinite(got).all()
