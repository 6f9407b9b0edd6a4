"""GPU parity of the grouped-query decode attention against the oracle.

turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step,
encode_attention_decode (f16 operands on Metal, scale 1/sqrt(head_dim), the
causal prefix [0, position]).  The output is one rounding of the exact value
up to fp32 noise: every stored element must be the nearest-even rounding of
the oracle's f64 value within 1e-5 of max |out| (check_f16_output /
check_bf16_output).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import quantized_transformer_decode_amd as qd
import synth
from helpers import DEV, check_bf16_output, check_f16_output

pytestmark = pytest.mark.gpu


def _to_f64(bits, f16):
    if f16:
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _dev16(bits, f16):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16).copy()).to(DEV)
    return t.view(torch.float16 if f16 else torch.bfloat16)


def _run(qb, kb, vb, heads, kv_heads, d, length, kv_start, scale, f16):
    q, k, v = (_dev16(a, f16) for a in (qb, kb, vb))
    out = torch.full((heads, d), float("nan"), dtype=q.dtype, device=DEV)
    ws, wsb = _workspace(heads, kv_heads, d)
    qd.attention_decode(q, k, v, heads, kv_heads, d, length, kv_start, scale, out, ws, wsb,
                        f16=f16)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _workspace(heads, kv_heads, d):
    """NaN-filled: no call may read a partial it did not write."""
    wsb = qd.attention_decode_workspace_bytes(heads, kv_heads, d)
    ws = torch.full((wsb // 4,), float("nan"), dtype=torch.float32, device=DEV)
    return ws, wsb


def _case(heads, kv_heads, d, rows, length, kv_start, f16, scale=None, key=0):
    print(f"attention heads={heads} kv={kv_heads} d={d} rows={rows} len={length} "
          f"start={kv_start} f16={f16}", flush=True)
    qb, kb, vb = synth.attention_inputs(heads, kv_heads, d, rows, key=(11, key, length), f16=f16)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    got = _run(qb, kb, vb, heads, kv_heads, d, length, kv_start, scale, f16)
    ref = oracle.attention_decode(_to_f64(qb, f16), _to_f64(kb, f16), _to_f64(vb, f16),
                                  length, scale, kv_start)
    check = check_f16_output if f16 else check_bf16_output
    check(got, ref, f"attention h={heads} kv={kv_heads} d={d} len={length} start={kv_start}")
    return got, (qb, kb, vb)


# Qwen3 0.6B/1.7B (16/8 heads), 4B (32/8), 8 query heads per K/V head, plain
# multi-head at d 64; windows of one row, within the single-chunk range
# (<= 128 rows), one past it, ragged multi-chunk lengths and long contexts
CASES = [
    (16, 8, 128, 1, 0), (16, 8, 128, 7, 0), (16, 8, 128, 128, 0), (16, 8, 128, 129, 0),
    (16, 8, 128, 33, 0),
    (16, 8, 128, 1000, 0), (16, 8, 128, 4097, 0), (32, 8, 128, 1500, 3),
    (64, 8, 128, 257, 0), (8, 8, 64, 333, 10), (4, 2, 64, 70000, 0), (16, 8, 128, 32768, 0),
]


@pytest.mark.parametrize("heads,kv_heads,d,length,kv_start", CASES)
@pytest.mark.parametrize("f16", [True, False])
def test_attention_parity(heads, kv_heads, d, length, kv_start, f16):
    _case(heads, kv_heads, d, length + 5, length, kv_start, f16)


def test_attention_one_row_is_that_row():
    # a single attended row has weight exactly 1: the output is that V row, bit for bit
    for f16 in (True, False):
        got, (_, _, vb) = _case(16, 8, 128, 9, 6, 5, f16)
        v = _to_f64(vb, f16)[5]                       # [kv_heads, d]
        assert np.array_equal(got, np.repeat(v, 2, axis=0))


def test_attention_peaked_and_flat():
    # scale 1 makes the scores ~N(0, 128): nearly one-hot rows; scale 0 is a plain mean
    _case(16, 8, 128, 2000, 2000, 0, True, scale=1.0, key=1)
    _case(16, 8, 128, 2000, 2000, 0, True, scale=0.0, key=2)
    _case(16, 8, 128, 3000, 2999, 17, False, scale=1.0, key=3)


def test_attention_rows_outside_window_ignored():
    # rows before kv_start and from length on are poisoned with huge values;
    # the output must match the oracle on the window alone
    heads, kv_heads, d, length, start = 16, 8, 128, 900, 123
    qb, kb, vb = synth.attention_inputs(heads, kv_heads, d, length + 40, key=(11, 9, 9))
    for a in (kb, vb):
        a[:start] = np.float16(60000.0).view(np.uint16)
        a[length:] = np.float16(-60000.0).view(np.uint16)
    scale = 1.0 / math.sqrt(d)
    got = _run(qb, kb, vb, heads, kv_heads, d, length, start, scale, True)
    ref = oracle.attention_decode(_to_f64(qb, True), _to_f64(kb, True), _to_f64(vb, True),
                                  length, scale, start)
    check_f16_output(got, ref, "poisoned outside the window")


def test_attention_workspace_reuse_and_stream():
    # two calls on one workspace in stream order, the second shorter, on a
    # non-default stream; each must match its own oracle result
    heads, kv_heads, d = 16, 8, 128
    s = torch.cuda.Stream()
    qb, kb, vb = synth.attention_inputs(heads, kv_heads, d, 5000, key=(11, 7, 7))
    q, k, v = (_dev16(a, True) for a in (qb, kb, vb))
    ws, wsb = _workspace(heads, kv_heads, d)
    outs = [torch.empty((heads, d), dtype=torch.float16, device=DEV) for _ in range(2)]
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        qd.attention_decode(q, k, v, heads, kv_heads, d, 5000, 0, 0.0884, outs[0], ws, wsb,
                            stream=s)
        qd.attention_decode(q, k, v, heads, kv_heads, d, 700, 0, 0.0884, outs[1], ws, wsb,
                            stream=s)
    s.synchronize()
    for out, n in zip(outs, (5000, 700)):
        ref = oracle.attention_decode(_to_f64(qb, True), _to_f64(kb, True), _to_f64(vb, True),
                                      n, 0.0884)
        check_f16_output(out.float().cpu().numpy().astype(np.float64), ref, f"reuse len={n}")


def test_attention_many_calls_one_workspace():
    # a decode loop: the window grows by one row per call (chunk counts and
    # rows per chunk change along the way) on one workspace; every call must
    # match the oracle
    heads, kv_heads, d = 16, 8, 128
    qb, kb, vb = synth.attention_inputs(heads, kv_heads, d, 600, key=(11, 8, 8))
    q, k, v = (_dev16(a, True) for a in (qb, kb, vb))
    ws, wsb = _workspace(heads, kv_heads, d)
    lengths = list(range(1, 80)) + list(range(250, 600, 37))
    outs = torch.empty((len(lengths), heads, d), dtype=torch.float16, device=DEV)
    for i, n in enumerate(lengths):
        qd.attention_decode(q, k, v, heads, kv_heads, d, n, 0, 0.0884, outs[i], ws, wsb)
    torch.cuda.synchronize()
    got = outs.float().cpu().numpy().astype(np.float64)
    qf, kf, vf = (_to_f64(a, True) for a in (qb, kb, vb))
    for i, n in enumerate(lengths):
        check_f16_output(got[i], oracle.attention_decode(qf, kf, vf, n, 0.0884), f"len={n}")
