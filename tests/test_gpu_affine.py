"""GPU parity of the affine-INT8 g64 loader and GEMV against the oracle.

turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs -- load_packed_linear
(blob), embed_row_bytes (dequant), Qwen3AsrMetalEngine::gemv / step (GEMV).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_transformer_decode_amd as qd
import synth
from helpers import (DEV, check_bf16_output, dev_bf16, host_bf16_bits, host_bf16_f64,
                     pack_on_device)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols", [(1, 64), (3, 192), (1024, 1024), (2048, 6144)])
def test_pack_bit_exact(rows, cols):
    print(f"pack rows={rows} cols={cols}", flush=True)
    tr = synth.affine_triplet(rows, cols, key=(1, rows, cols))
    blob = pack_on_device(tr)
    torch.cuda.synchronize()
    want = oracle.affine_pack(tr.codes, tr.scales, tr.biases, rows, cols)
    assert np.array_equal(blob.cpu().numpy(), want)


def _run_gemv(tr, blob, x_bits, m):
    x = dev_bf16(x_bits)
    y = torch.full((m, tr.rows), float("nan"), dtype=torch.bfloat16, device=DEV)
    qd.qgemv_affine_i8_g64(blob, tr.rows, tr.cols, x, y, m)
    torch.cuda.synchronize()
    return y


# (rows, cols, m): tiny and ragged rows, several waves' worth of rows, the
# 1024x1024 single-GEMV workload, each decode-step shape, tokens 1..16
CASES = [
    (1, 64, 1), (5, 128, 3), (17, 64, 16), (130, 192, 2), (1024, 1024, 1),
    (2048, 1024, 1), (1024, 2048, 1), (3072, 1024, 1), (1024, 3072, 1),
    (1000, 2048, 4), (6144, 2048, 10), (2048, 6144, 16), (333, 320, 7),
    # the widest input the GEMV takes (8192 columns) at 1 and 16 tokens
    (64, 8192, 1), (257, 8192, 16),
]


@pytest.mark.parametrize("rows,cols,m", CASES)
def test_gemv_parity(rows, cols, m):
    print(f"affine gemv rows={rows} cols={cols} m={m}", flush=True)
    tr = synth.affine_triplet(rows, cols, key=(1, rows, cols))
    blob = pack_on_device(tr)
    x = synth.x_bf16(m, cols, key=(1, rows, cols + m))
    y = _run_gemv(tr, blob, x, m)
    ref = oracle.affine_gemv(blob.cpu().numpy(), rows, cols, x)
    check_bf16_output(host_bf16_f64(y), ref, f"{rows}x{cols} m={m}")


def test_lm_head_full_size_sampled():
    # tied LM head 151936 x 1024 at batch 1, checked on sampled rows
    rows, cols = 151936, 1024
    print("affine gemv lm head", flush=True)
    tr = synth.affine_triplet(rows, cols, key=(3, 28, 7))
    blob = pack_on_device(tr)
    x = synth.x_bf16(1, cols, key=(3, 28, 8))
    y = host_bf16_f64(_run_gemv(tr, blob, x, 1))
    sel = np.unique(np.concatenate([np.random.default_rng(0).integers(0, rows, 2048),
                                    [0, 1, rows - 2, rows - 1]]))
    ref = oracle.affine_gemv(blob.cpu().numpy(), rows, cols, x, row_sel=sel)
    check_bf16_output(y[:, sel], ref, "lm head")


# Large matrices on sampled rows, one per kernel path: the batch-1 VALU
# streaming kernel (151936 x 2048), the matrix-core streaming walk with x in
# LDS (LM head at M=16), without chunked scales (cols % 256 != 0), and with x
# too large for LDS (M=16, 4608 columns).
BIG = [(151936, 2048, 1), (151936, 1024, 16), (65536, 320, 4), (65600, 4608, 16)]


@pytest.mark.parametrize("rows,cols,m", BIG)
def test_large_sampled(rows, cols, m):
    print(f"affine gemv sampled rows={rows} cols={cols} m={m}", flush=True)
    tr = synth.affine_triplet(rows, cols, key=(6, rows, cols))
    blob = pack_on_device(tr)
    x = synth.x_bf16(m, cols, key=(6, rows, cols + m))
    y = host_bf16_f64(_run_gemv(tr, blob, x, m))
    sel = np.unique(np.concatenate([np.random.default_rng(1).integers(0, rows, 1024),
                                    np.arange(16), np.arange(rows - 40, rows)]))
    ref = oracle.affine_gemv(blob.cpu().numpy(), rows, cols, x, row_sel=sel)
    check_bf16_output(y[:, sel], ref, f"{rows}x{cols} m={m} sampled")
    del blob


# Same-input groups in one launch: the decode step's q/k/v and gate/up, ragged
# row counts, the per-group scale path (cols % 256 != 0), four matrices, and a
# group large enough for the streaming walk to cross matrix boundaries
# (checked on sampled rows).
GROUPS = [
    ((2048, 1024, 1024), 1024, 1), ((6144, 6144), 2048, 16), ((17, 130, 64, 5), 192, 3),
    ((1000, 33), 2048, 10), ((40000, 30016), 1024, 4),
]


@pytest.mark.parametrize("rows_list,cols,m", GROUPS)
def test_group_parity(rows_list, cols, m):
    print(f"affine group rows={rows_list} cols={cols} m={m}", flush=True)
    trs = [synth.affine_triplet(r, cols, key=(7, k, r)) for k, r in enumerate(rows_list)]
    blobs = [pack_on_device(tr) for tr in trs]
    x = synth.x_bf16(m, cols, key=(7, cols, m))
    ys = [torch.full((m, r), float("nan"), dtype=torch.bfloat16, device=DEV) for r in rows_list]
    qd.qgemv_affine_i8_g64_group([(b, y, r) for b, y, r in zip(blobs, ys, rows_list)],
                                 cols, dev_bf16(x), m)
    torch.cuda.synchronize()
    for k, (r, b, y) in enumerate(zip(rows_list, blobs, ys)):
        got = host_bf16_f64(y)
        if r > 4096:
            sel = np.unique(np.concatenate([np.random.default_rng(k).integers(0, r, 512),
                                            np.arange(16), np.arange(r - 24, r)]))
            ref = oracle.affine_gemv(b.cpu().numpy(), r, cols, x, row_sel=sel)
            check_bf16_output(got[:, sel], ref, f"group item {k} ({r}x{cols}) sampled")
        else:
            ref = oracle.affine_gemv(b.cpu().numpy(), r, cols, x)
            check_bf16_output(got, ref, f"group item {k} ({r}x{cols})")


def test_closed_forms_on_device():
    # zero scales: y = sum_g bias_g * X_g; constant codes q0: y = sum_g
    # (s_g q0 + b_g) X_g -- compared with the oracle, which is pinned to
    # these closed forms on the CPU
    rows, cols, m = 96, 512, 3
    tr = synth.affine_triplet(rows, cols, key=(9, 0, 0))
    tr.scales[:] = 0
    x = synth.x_bf16(m, cols, key=(9, 0, 1))
    blob = pack_on_device(tr)
    y = host_bf16_f64(_run_gemv(tr, blob, x, m))
    check_bf16_output(y, oracle.affine_gemv(blob.cpu().numpy(), rows, cols, x), "zero scale")
    tr = synth.affine_triplet(rows, cols, key=(9, 0, 2))
    tr.codes[:] = np.uint32(255 * 0x01010101)
    blob = pack_on_device(tr)
    y = host_bf16_f64(_run_gemv(tr, blob, x, m))
    check_bf16_output(y, oracle.affine_gemv(blob.cpu().numpy(), rows, cols, x), "const code")


def test_brute_force_k64_exact():
    codes = np.arange(64, dtype=np.uint8).reshape(1, 64)
    tr = synth.affine_triplet_custom(codes, np.array([[2.0 ** -8]]), np.array([[-0.5]]))
    blob = pack_on_device(tr)
    x = synth.to_bf16_bits(np.ones((1, 64), dtype=np.float32))
    y = host_bf16_f64(_run_gemv(tr, blob, x, 1))
    assert y[0, 0] == -24.125


def test_output_at_offset_and_untouched_neighbours():
    # y may sit inside a larger buffer (a K/V cache row): only [m, rows]
    # elements at the offset are written
    rows, cols = 64, 256
    tr = synth.affine_triplet(rows, cols, key=(10, 0, 0))
    blob = pack_on_device(tr)
    x = dev_bf16(synth.x_bf16(1, cols, key=(10, 0, 1)))
    buf = torch.full((3 * rows + 1,), 7.0, dtype=torch.bfloat16, device=DEV)
    out = buf[rows + 1: 2 * rows + 1]
    qd.qgemv_affine_i8_g64(blob, rows, cols, x, out, 1)
    torch.cuda.synchronize()
    b = buf.float().cpu().numpy()
    assert np.all(b[: rows + 1] == 7.0) and np.all(b[2 * rows + 1:] == 7.0)
    ref = oracle.affine_gemv(blob.cpu().numpy(), rows, cols, host_bf16_bits(x.view(1, cols)))
    check_bf16_output(b[rows + 1: 2 * rows + 1].reshape(1, rows).astype(np.float64), ref, "offset")


def test_invalid_args_raise_without_launch():
    with pytest.raises(qd.QDError) as e:
        t = torch.empty(16, dtype=torch.uint8, device=DEV)
        qd.qgemv_affine_i8_g64(t, 1, 100, t, t, 1)
    assert e.value.status == qd.QD_ESHAPE
