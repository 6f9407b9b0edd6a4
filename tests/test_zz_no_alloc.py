"""GPU test of the allocation-free attention entry point
(attention_decode_noalloc): its output against attention_decode's on the
same inputs, bit for bit (the same kernels; only where the chunk partials
live differs), and against the oracle (f16 outputs the nearest-even rounding
of the exact attention within 1e-5 of max |out|) -- on two calls in a row,
the second with a smaller window and fewer heads, so the second reads a
scratch array that still holds the first call's partials.

turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step,
encode_attention_decode over rows [0, position].
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_transformer_decode_amd as qd
import synth
from helpers import DEV, check_f16_output, dev_f16

pytestmark = pytest.mark.gpu


def _h(t):
    return t.float().cpu().numpy().astype(np.float64)


def _bits(b):
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("first,second", [
    ((16, 8, 128, 20000), (16, 8, 128, 777)),     # Qwen3-0.6B heads, long then short window
    ((32, 8, 128, 70000), (4, 2, 64, 129)),       # more chunks, then fewer heads and d 64
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for call, (heads, kvh, d, n) in enumerate((first, second)):
        print(f"attention_decode_noalloc call {call}: heads={heads} kv={kvh} d={d} rows={n}",
              flush=True)
        qb, kb, vb = synth.attention_inputs(heads, kvh, d, n, key=(70, call, heads))
        q, k, v = dev_f16(qb), dev_f16(kb), dev_f16(vb)
        scale = float(np.float32(1.0) / np.sqrt(np.float32(d)))
        wsb = qd.attention_decode_workspace_bytes(heads, kvh, d)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        out_ws = torch.full((heads, d), float("nan"), dtype=torch.float16, device=DEV)
        out_na = torch.full((heads, d), float("nan"), dtype=torch.float16, device=DEV)
        qd.attention_decode(q, k, v, heads, kvh, d, n, 0, scale, out_ws, ws, wsb)
        qd.attention_decode_noalloc(q, k, v, heads, kvh, d, n, 0, scale, out_na)
        torch.cuda.synchronize()
        assert torch.equal(out_ws.view(torch.int16), out_na.view(torch.int16))
        ref = oracle.attention_decode(_bits(qb).reshape(heads, d),
                                      _bits(kb).reshape(n, kvh, d),
                                      _bits(vb).reshape(n, kvh, d), n, scale)
        check_f16_output(_h(out_na), ref, f"call {call}")


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    q = torch.zeros((8192, 128), dtype=torch.float16, device=DEV)
    kv = torch.zeros((1, 1024, 128), dtype=torch.float16, device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(qd.QDError) as ei:
        qd.attention_decode_noalloc(q, kv, kv, 8192, 1024, 128, 1, 0, 0.088, out)
    assert ei.value.status == qd.QD_ESCRATCH
