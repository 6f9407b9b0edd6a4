"""GPU parity of the f16-activation affine GEMV and of the tied-embedding
row lookup against the oracle.

turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::gemv
(f16 activations on Metal), embed_row_bytes (f32 q*scale + bias, stored f16).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_transformer_decode_amd as qd
import synth
from helpers import DEV, check_f16_output, dev_f16, pack_on_device

pytestmark = pytest.mark.gpu


def _gemv_f16(blob, rows, cols, x_bits, m):
    y = torch.full((m, rows), float("nan"), dtype=torch.float16, device=DEV)
    qd.qgemv_affine_i8_g64_f16(blob, rows, cols, dev_f16(x_bits), y, m)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


# tiny and ragged rows, each decode-step width, tokens 1..16, the widest input
CASES = [(1, 64, 1), (17, 64, 16), (130, 192, 2), (1024, 1024, 1), (2048, 1024, 4),
         (1024, 3072, 1), (333, 320, 7), (6144, 2048, 10), (257, 8192, 16)]


@pytest.mark.parametrize("rows,cols,m", CASES)
def test_gemv_f16_parity(rows, cols, m):
    print(f"affine gemv f16 rows={rows} cols={cols} m={m}", flush=True)
    tr = synth.affine_triplet(rows, cols, key=(9, rows, cols))
    blob = pack_on_device(tr)
    x = synth.x_f16(m, cols, key=(9, rows, cols + m))
    y = _gemv_f16(blob, rows, cols, x, m)
    ref = oracle.affine_gemv(blob.cpu().numpy(), rows, cols, x, x_f16=True)
    check_f16_output(y, ref, f"f16 {rows}x{cols} m={m}")


@pytest.mark.parametrize("m", [1, 16])
def test_gemv_f16_lm_head_sampled(m):
    rows, cols = 151936, 1024
    print(f"affine gemv f16 lm head m={m}", flush=True)
    tr = synth.affine_triplet(rows, cols, key=(9, 28, 7))
    blob = pack_on_device(tr)
    x = synth.x_f16(m, cols, key=(9, 28, 8 + m))
    y = _gemv_f16(blob, rows, cols, x, m)
    sel = np.unique(np.concatenate([np.random.default_rng(2).integers(0, rows, 1024),
                                    [0, 1, rows - 2, rows - 1]]))
    ref = oracle.affine_gemv(blob.cpu().numpy(), rows, cols, x, row_sel=sel, x_f16=True)
    check_f16_output(y[:, sel], ref, "f16 lm head")


def test_gemv_f16_brute_force_exact():
    # q_c = c, x_c = 1, s = 2^-8, b = -0.5 -> exactly -24.125 (an f16 value)
    codes = np.arange(64, dtype=np.uint8).reshape(1, 64)
    tr = synth.affine_triplet_custom(codes, np.array([[2.0 ** -8]]), np.array([[-0.5]]))
    blob = pack_on_device(tr)
    y = _gemv_f16(blob, 1, 64, np.full((1, 64), 0x3C00, dtype=np.uint16), 1)
    assert y[0, 0] == -24.125


def _embed(blob, rows, cols, ids, f16):
    out = torch.full((len(ids), cols), -1, dtype=torch.int16, device=DEV)
    qd.affine_i8_g64_embed_rows(blob, rows, cols, ids, out, out_f16=f16)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("rows,cols", [(151936, 1024), (4096, 2048), (7, 64), (300, 8192)])
@pytest.mark.parametrize("f16", [True, False])
def test_embed_rows_bit_exact(rows, cols, f16):
    print(f"embed rows {rows}x{cols} f16={f16}", flush=True)
    tr = synth.affine_triplet(rows, cols, key=(10, rows, cols))
    blob = pack_on_device(tr)
    host = blob.cpu().numpy()
    rng = np.random.default_rng(rows + cols)
    ids = [0, rows - 1] + [int(t) for t in rng.integers(0, rows, 14)]
    for n in (1, 3, 16):
        got = _embed(blob, rows, cols, ids[:n], f16)
        for i, t in enumerate(ids[:n]):
            assert np.array_equal(got[i], oracle.affine_embed_row(host, rows, cols, t, f16)), \
                f"token {t}"


def test_embed_row_double_rounding_on_device():
    # f32 first, then f16: 1 + 2^-11 + 2^-25 -> 0x3C00 (not 0x3C01)
    cols = 64
    tr = synth.affine_triplet_custom(np.full((1, cols), 226, dtype=np.uint8),
                                     np.array([[145 * 2.0 ** -26]]), np.array([[1.0]]))
    blob = pack_on_device(tr)
    assert np.all(_embed(blob, 1, cols, [0], True) == 0x3C00)
    assert np.all(_embed(blob, 1, cols, [0], False) == 0x3F80)
