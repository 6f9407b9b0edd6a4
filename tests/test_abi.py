"""CPU tests of the C ABI: the library loads, exports every function that
include/qdecode.h declares, computes the layout helpers, and rejects every
invalid argument with the documented status before touching the GPU.

Pointers passed here are fake (never dereferenced): validation runs on the
host before any HIP call.  The one test that gets past validation runs only
where no GPU is visible, so the call stops at the device check.
"""
import ctypes
import os
import re

import pytest

import quantized_transformer_decode_amd as qd
from conftest import ROOT

P = ctypes.c_void_p
A = 0x7f0000000000  # fake, 256-byte aligned device address
B = 0x7f1000000000
C = 0x7f2000000000


def _declared():
    with open(os.path.join(ROOT, "include", "qdecode.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"}


def test_header_symbols_exported():
    L = qd.lib()
    names = _declared()
    assert names == set(qd.EXPORTS), names ^ set(qd.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    L = qd.lib()
    for s in range(6):
        assert L.qd_status_string(s).decode().startswith(
            ["QD_OK", "QD_EINVAL", "QD_ESHAPE", "QD_EALIGN", "QD_EDEVICE", "QD_EHIP"][s])
    assert L.qd_status_string(99) == b"QD_UNKNOWN"
    assert b"gfx950" in L.qd_version()
    assert L.qd_last_hip_error() == 0


def test_layout_helpers():
    # turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- PackedLinear::resident
    assert qd.affine_i8_g64_scales_offset(1024, 1024) == 1048576
    assert qd.affine_i8_g64_biases_offset(1024, 1024) == 1048576 + 32768
    assert qd.affine_i8_g64_bytes(1024, 1024) == 1114112
    assert qd.affine_i8_g64_bytes(151936, 1024) == 155582464 + 2 * 4861952
    assert qd.affine_i8_g64_bytes(1024, 100) == 0
    assert qd.affine_i8_g64_bytes(0, 64) == 0
    # fuel-transformers 0.19.1, lazy_quantized_whisper.rs -- 18-byte blocks
    # padded to a multiple of 4
    assert qd.q4_0_bytes(1, 32) == 20
    assert qd.q4_0_bytes(2, 32) == 36
    assert qd.q4_0_bytes(2048, 512) == 589824
    assert qd.q4_0_bytes(1, 48) == 0


def _call(fn, *args):
    return getattr(qd.lib(), fn)(*args)


def test_errors_affine_gemv():
    f = "qgemv_affine_i8_g64"
    ok = (A, 64, 1024, B, C, 1, None)
    assert _call(f, None, 64, 1024, B, C, 1, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, None, C, 1, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, B, None, 1, None) == qd.QD_EINVAL
    assert _call(f, A, 0, 1024, B, C, 1, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, B, C, 0, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, B, C, 17, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1000, B, C, 1, None) == qd.QD_ESHAPE
    assert _call(f, A, 64, 32, B, C, 1, None) == qd.QD_ESHAPE
    assert _call(f, A, 64, 16384, B, C, 1, None) == qd.QD_ESHAPE
    assert _call(f, A + 8, 64, 1024, B, C, 1, None) == qd.QD_EALIGN
    assert _call(f, A, 64, 1024, B + 2, C, 1, None) == qd.QD_EALIGN
    assert _call(f, A, 64, 1024, B, C + 1, 1, None) == qd.QD_EALIGN
    # output overlapping the weights or x
    assert _call(f, A, 64, 1024, B, A + 64, 1, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, B, B + 2, 1, None) == qd.QD_EINVAL
    assert ok  # the valid form is exercised by test_valid_args_reach_device_check


def test_errors_affine_gemv_f16():
    # the f16 variant validates exactly like the BF16 one
    f = "qgemv_affine_i8_g64_f16"
    assert _call(f, None, 64, 1024, B, C, 1, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, B, C, 17, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1000, B, C, 1, None) == qd.QD_ESHAPE
    assert _call(f, A, 64, 1024, B + 2, C, 1, None) == qd.QD_EALIGN
    assert _call(f, A, 64, 1024, B, A + 64, 1, None) == qd.QD_EINVAL


def _ids(*v):
    return (ctypes.c_int64 * len(v))(*v)


def test_errors_embed_rows():
    f = "affine_i8_g64_embed_rows"
    ids = _ids(0, 5, 63)
    assert _call(f, None, 64, 1024, ids, 3, C, 1, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, None, 3, C, 1, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, ids, 3, None, 1, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, ids, 0, C, 1, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, _ids(*range(17)), 17, C, 1, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, ids, 3, C, 2, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1024, _ids(0, 64), 2, C, 1, None) == qd.QD_EINVAL  # id >= rows
    assert _call(f, A, 64, 1024, _ids(-1), 1, C, 0, None) == qd.QD_EINVAL
    assert _call(f, A, 64, 1000, ids, 3, C, 1, None) == qd.QD_ESHAPE
    assert _call(f, A + 8, 64, 1024, ids, 3, C, 1, None) == qd.QD_EALIGN
    assert _call(f, A, 64, 1024, ids, 3, C + 4, 1, None) == qd.QD_EALIGN
    assert _call(f, A, 64, 1024, ids, 3, A + 128, 1, None) == qd.QD_EINVAL  # overlaps the blob


def _lin(*items):
    arr = (qd.Q40LinearItem * len(items))()
    for k, (w, b, y, r) in enumerate(items):
        arr[k] = qd.Q40LinearItem(w, b, y, r)
    return arr


def test_errors_qlinear():
    for f, y_al in (("qlinear_q4_0_gemv", 4), ("qlinear_q4_0_gemm", 16)):
        D = 0x7f3000000000
        ok = _lin((A, D, C, 64))
        assert _call(f, None, 1, 512, B, 4, 0, None) == qd.QD_EINVAL
        assert _call(f, ok, 0, 512, B, 4, 0, None) == qd.QD_EINVAL
        assert _call(f, ok, 1, 512, B, 4, 2, None) == qd.QD_EINVAL        # gelu not 0/1
        assert _call(f, ok, 1, 500, B, 4, 0, None) == qd.QD_ESHAPE
        assert _call(f, _lin((A, D + 2, C, 64)), 1, 512, B, 4, 0, None) == qd.QD_EALIGN
        assert _call(f, _lin((A, D, C + y_al // 2, 64)), 1, 512, B, 4, 0, None) == qd.QD_EALIGN
        # output overlapping a bias, weights or another output
        assert _call(f, _lin((A, D, D + 16, 64)), 1, 512, B, 4, 0, None) == qd.QD_EINVAL
        assert _call(f, _lin((A, None, A + 64, 64)), 1, 512, B, 4, 0, None) == qd.QD_EINVAL
        assert _call(f, _lin((A, None, C, 64), (A, None, C + 256, 64)), 2, 512, B, 4, 0,
                     None) == qd.QD_EINVAL
    assert _call("qlinear_q4_0_gemv", _lin((A, None, C, 64)), 1, 512, B, 17, 0,
                 None) == qd.QD_EINVAL


def test_errors_q4_0_gemv_and_gemm():
    for f in ("qgemv_q4_0", "qgemm_q4_0_prefill"):
        assert _call(f, None, 64, 512, B, C, 1, None) == qd.QD_EINVAL
        assert _call(f, A, 64, 512, None, C, 1, None) == qd.QD_EINVAL
        assert _call(f, A, 64, 512, B, None, 1, None) == qd.QD_EINVAL
        assert _call(f, A, -1, 512, B, C, 1, None) == qd.QD_EINVAL
        assert _call(f, A, 64, 512, B, C, 0, None) == qd.QD_EINVAL
        assert _call(f, A, 64, 480, B, C, 1, None) == qd.QD_ESHAPE   # % 256
        assert _call(f, A, 64, 128, B, C, 1, None) == qd.QD_ESHAPE
        assert _call(f, A + 4, 64, 512, B, C, 1, None) == qd.QD_EALIGN
        assert _call(f, A, 64, 512, B + 4, C, 1, None) == qd.QD_EALIGN
        assert _call(f, A, 64, 512, B, C + 2, 1, None) == qd.QD_EALIGN
        assert _call(f, A, 64, 512, B, B, 1, None) == qd.QD_EINVAL
    assert _call("qgemv_q4_0", A, 64, 512, B, C, 17, None) == qd.QD_EINVAL
    assert _call("qgemm_q4_0_prefill", A, 64, 512, B, C + 4, 1, None) == qd.QD_EALIGN
    assert _call("qgemm_q4_0_prefill", A, 64, 512, B, C, (1 << 22) + 1, None) == qd.QD_EINVAL


D = 0x7f3000000000
E = 0x7f4000000000


def _affine_items(*items):
    arr = (qd.AffineGemvItem * max(1, len(items)))()
    for i, (w, y, rows) in enumerate(items):
        arr[i] = qd.AffineGemvItem(w, y, rows)
    return arr


def _q4_items(*items):
    arr = (qd.Q40GemvItem * max(1, len(items)))()
    for i, (w, y, rows) in enumerate(items):
        arr[i] = qd.Q40GemvItem(w, y, rows)
    return arr


def test_errors_affine_gemv_group():
    f = "qgemv_affine_i8_g64_group"
    two = _affine_items((A, C, 64), (D, E, 32))
    assert _call(f, None, 1, 1024, B, 1, None) == qd.QD_EINVAL
    assert _call(f, two, 0, 1024, B, 1, None) == qd.QD_EINVAL
    five = _affine_items(*[(A + (i << 32), C + (i << 32), 16) for i in range(5)])
    assert _call(f, five, 5, 1024, B, 1, None) == qd.QD_EINVAL      # at most 4
    assert _call(f, two, 2, 1024, None, 1, None) == qd.QD_EINVAL
    assert _call(f, two, 2, 1024, B, 17, None) == qd.QD_EINVAL
    assert _call(f, two, 2, 1000, B, 1, None) == qd.QD_ESHAPE
    assert _call(f, _affine_items((A, C, 64), (None, E, 32)), 2, 1024, B, 1, None) == qd.QD_EINVAL
    assert _call(f, _affine_items((A, C, 64), (D, E, 0)), 2, 1024, B, 1, None) == qd.QD_EINVAL
    assert _call(f, _affine_items((A, C, 64), (D + 8, E, 32)), 2, 1024, B, 1, None) == qd.QD_EALIGN
    assert _call(f, two, 2, 1024, B + 2, 1, None) == qd.QD_EALIGN
    # an output over another item's weights, over another output, over x
    assert _call(f, _affine_items((A, C, 64), (D, A + 64, 32)), 2, 1024, B, 1, None) == qd.QD_EINVAL
    assert _call(f, _affine_items((A, C, 64), (D, C + 64, 32)), 2, 1024, B, 1, None) == qd.QD_EINVAL
    assert _call(f, _affine_items((A, B + 2, 64), (D, E, 32)), 2, 1024, B, 1, None) == qd.QD_EINVAL


def test_errors_q4_0_gemv_group():
    f = "qgemv_q4_0_group"
    two = _q4_items((A, C, 64), (D, E, 32))
    assert _call(f, None, 1, 512, B, 1, None) == qd.QD_EINVAL
    assert _call(f, two, 0, 512, B, 1, None) == qd.QD_EINVAL
    assert _call(f, two, 5, 512, B, 1, None) == qd.QD_EINVAL
    assert _call(f, two, 2, 512, B, 0, None) == qd.QD_EINVAL
    assert _call(f, two, 2, 480, B, 1, None) == qd.QD_ESHAPE
    assert _call(f, _q4_items((A, C, 64), (D, E + 2, 32)), 2, 512, B, 1, None) == qd.QD_EALIGN
    assert _call(f, two, 2, 512, B + 4, 1, None) == qd.QD_EALIGN
    assert _call(f, _q4_items((A, C, 64), (D, A + 64, 32)), 2, 512, B, 1, None) == qd.QD_EINVAL
    assert _call(f, _q4_items((A, C, 64), (D, C + 128, 32)), 2, 512, B, 1, None) == qd.QD_EINVAL


def test_errors_quantize_and_pack():
    f = "q4_0_quantize"
    assert _call(f, None, 4, 64, C, None) == qd.QD_EINVAL
    assert _call(f, A, 4, 64, None, None) == qd.QD_EINVAL
    assert _call(f, A, 0, 64, C, None) == qd.QD_EINVAL
    assert _call(f, A, 4, 48, C, None) == qd.QD_ESHAPE
    assert _call(f, A + 4, 4, 64, C, None) == qd.QD_EALIGN
    assert _call(f, A, 4, 64, C + 2, None) == qd.QD_EALIGN
    assert _call(f, A, 4, 64, A + 16, None) == qd.QD_EINVAL
    g = "affine_i8_g64_pack"
    assert _call(g, None, B, C, 4, 64, A, None) == qd.QD_EINVAL
    assert _call(g, A, B, C, 4, 96, A + (1 << 20), None) == qd.QD_ESHAPE
    assert _call(g, A, B, C, 4, 64, A + (1 << 20) + 8, None) == qd.QD_EALIGN
    assert _call(g, A, B, C, 4, 64, A + 128, None) == qd.QD_EINVAL  # overlaps codes


def test_errors_stream_read():
    f = "qd_stream_read"
    assert _call(f, None, 1024, B, None) == qd.QD_EINVAL
    assert _call(f, A, 1024, None, None) == qd.QD_EINVAL
    assert _call(f, A, 0, B, None) == qd.QD_EINVAL
    assert _call(f, A, 1000, B, None) == qd.QD_ESHAPE
    assert _call(f, A + 8, 1024, B, None) == qd.QD_EALIGN
    assert _call(f, A, 1024, B + 2, None) == qd.QD_EALIGN


OUT = 0x7f3000000000
WS = 0x7f4000000000


def test_attention_workspace_bytes():
    f = qd.attention_decode_workspace_bytes
    # one float per (head, chunk, d + 2) for at most ceil(512 / kv_heads) chunks
    assert f(16, 8, 128) == 16 * 64 * 130 * 4
    assert f(8, 8, 64) == 8 * 64 * 66 * 4
    assert f(65, 65, 128) == 65 * 8 * 130 * 4
    assert f(8, 1, 128) == 8 * 512 * 130 * 4
    assert f(16, 8, 96) == 0          # head_dim
    assert f(24, 8, 128) == 0         # group of 3
    assert f(16, 0, 128) == 0
    assert f(16, 16, 128) > 0 and f(128, 16, 128) > 0 and f(256, 16, 128) == 0


def test_errors_attention_decode():
    f = "attention_decode"
    ws = qd.attention_decode_workspace_bytes(16, 8, 128)

    def call(q=A, k=B, v=C, heads=16, kvh=8, d=128, n=100, s=0, scale=0.088, f16=1, out=OUT,
             w=WS, wb=ws):
        return _call(f, q, k, v, heads, kvh, d, n, s, ctypes.c_float(scale), f16, out, w, wb,
                     None)

    for bad in ({"q": None}, {"k": None}, {"v": None}, {"out": None}, {"w": None}):
        assert call(**bad) == qd.QD_EINVAL
    assert call(f16=2) == qd.QD_EINVAL
    assert call(heads=24) == qd.QD_ESHAPE             # group of 3
    assert call(heads=12) == qd.QD_ESHAPE             # not a multiple of kv_heads
    assert call(heads=256, kvh=16) == qd.QD_ESHAPE    # group of 16
    assert call(d=96) == qd.QD_ESHAPE
    assert call(kvh=0) == qd.QD_ESHAPE
    assert call(n=0) == qd.QD_EINVAL                  # empty window
    assert call(s=100) == qd.QD_EINVAL
    assert call(s=-1) == qd.QD_EINVAL
    assert call(n=(1 << 30) + 1, wb=1 << 40) == qd.QD_EINVAL
    assert call(scale=float("nan")) == qd.QD_EINVAL
    assert call(scale=float("inf")) == qd.QD_EINVAL
    assert call(q=A + 8) == qd.QD_EALIGN
    assert call(k=B + 2) == qd.QD_EALIGN
    assert call(out=OUT + 8) == qd.QD_EALIGN
    assert call(w=WS + 4) == qd.QD_EALIGN
    assert call(wb=ws - 1) == qd.QD_EINVAL            # workspace too small
    assert call(out=B + 4096) == qd.QD_EINVAL         # output inside the K cache
    assert call(w=C + 4096) == qd.QD_EINVAL           # workspace inside the V cache
    assert call(out=WS + 256) == qd.QD_EINVAL         # output inside the workspace


def test_errors_decoder_ops():
    f = "rmsnorm_f16"
    F = ctypes.c_float
    assert _call(f, None, None, B, 1024, F(1e-6), C, None) == qd.QD_EINVAL
    assert _call(f, A, None, None, 1024, F(1e-6), C, None) == qd.QD_EINVAL
    assert _call(f, A, None, B, 1024, F(-1.0), C, None) == qd.QD_EINVAL
    assert _call(f, A, None, B, 1024, F(float("nan")), C, None) == qd.QD_EINVAL
    assert _call(f, A, None, B, 1000, F(1e-6), C, None) == qd.QD_ESHAPE
    assert _call(f, A, None, B, 16384, F(1e-6), C, None) == qd.QD_ESHAPE
    assert _call(f, A + 4, None, B, 1024, F(1e-6), C, None) == qd.QD_EALIGN
    assert _call(f, A, OUT + 2, B, 1024, F(1e-6), C, None) == qd.QD_EALIGN
    assert _call(f, A, None, B, 1024, F(1e-6), A + 64, None) == qd.QD_EINVAL  # out overlaps x

    f = "qk_norm_rope_f16"

    def qk(q=A, ks=B, vs=C, qn=OUT, kn=OUT + 256, h=16, kv=8, d=128, eps=1e-6, th=1e6,
           pos=WS, cap=4096, kc=0x7f5000000000, vc=0x7f6000000000, err=WS + 64):
        return _call(f, q, ks, vs, qn, kn, h, kv, d, F(eps), F(th), pos, cap, kc, vc, err, None)

    for bad in ({"q": None}, {"ks": None}, {"pos": None}, {"vc": None}, {"err": None}):
        assert qk(**bad) == qd.QD_EINVAL
    assert qk(d=96) == qd.QD_ESHAPE
    assert qk(kv=0) == qd.QD_ESHAPE
    assert qk(cap=0) == qd.QD_EINVAL
    assert qk(th=0.0) == qd.QD_EINVAL
    assert qk(eps=float("inf")) == qd.QD_EINVAL
    assert qk(q=A + 1) == qd.QD_EALIGN
    assert qk(pos=WS + 2) == qd.QD_EALIGN

    f = "silu_mul_f16"
    assert _call(f, None, B, C, 3072, None) == qd.QD_EINVAL
    assert _call(f, A, B, C, 3070, None) == qd.QD_ESHAPE
    assert _call(f, A, B, C, 0, None) == qd.QD_ESHAPE
    assert _call(f, A + 2, B, C, 3072, None) == qd.QD_EALIGN
    assert _call(f, A, B, B + 8, 3072, None) == qd.QD_EINVAL     # out overlaps up
    assert _call(f, A, B, A + 8, 3072, None) == qd.QD_EINVAL     # partly over gate


def _qwen3(**kw):
    layer = qd.Qwen3Layer(*[0x7f7000000000 + (i << 32) for i in range(13)])
    arr = (qd.Qwen3Layer * 2)(layer, layer)
    d = dict(hidden=1024, heads=16, kv_heads=8, head_dim=128, inter=3072, vocab=151936,
             n_layers=2, capacity=4096, eps=1e-6, theta=1e6, layers=arr,
             final_norm=0x7f8000000000, embed=0x7f9000000000)
    d.update(kw)
    m = qd.Qwen3Model(**d)
    m._keep = arr
    return m


def test_qwen3_step_workspace_and_errors():
    wb = qd.qwen3_step_workspace_bytes
    m = _qwen3()
    n = wb(m)
    # error word, normed, q, k, v, attn, delta, gate, up (each 256-padded),
    # attention partials, fp32 o-projection partial rows (one per K/V head)
    rows = 256 + 2048 + 4096 + 2048 + 2048 + 4096 + 2048 + 6144 + 6144
    # ... and the rotated q row
    assert n == rows + qd.attention_decode_workspace_bytes(16, 8, 128) + 8 * 1024 * 4 + 4096
    # more than 8 K/V heads: the o projection is its own GEMV, no partial rows
    # (q, attn 16 x 64 x 2; k, v 16 x 64 x 2: the same padded sizes as above)
    n16 = wb(_qwen3(heads=16, kv_heads=16, head_dim=64))
    rows16 = 256 + 2048 + 2048 + 2048 + 2048 + 2048 + 2048 + 6144 + 6144
    assert n16 == rows16 + qd.attention_decode_workspace_bytes(16, 16, 64) + 2048
    for bad in (dict(hidden=1000), dict(head_dim=96), dict(heads=24), dict(inter=16384),
                dict(capacity=0), dict(vocab=0), dict(n_layers=0)):
        assert wb(_qwen3(**bad)) == 0, bad
    f = "qwen3_step_run"
    X, POS, LOG = 0x7fa000000000, 0x7fb000000000, 0x7fc000000000
    ref = ctypes.byref

    def run(model=m, ws=WS, nb=n, x=X, pos=POS, logits=LOG, adv=1):
        return _call(f, ref(model), ws, nb, x, pos, logits, adv, None)

    assert run(ws=None) == qd.QD_EINVAL
    assert run(x=None) == qd.QD_EINVAL
    assert run(pos=None) == qd.QD_EINVAL
    assert run(adv=2) == qd.QD_EINVAL
    assert run(nb=n - 1) == qd.QD_EINVAL
    assert run(model=_qwen3(embed=None)) == qd.QD_EINVAL
    assert run(model=_qwen3(theta=-1.0)) == qd.QD_EINVAL
    assert run(model=_qwen3(hidden=1000)) == qd.QD_ESHAPE
    assert run(ws=WS + 16) == qd.QD_EALIGN
    assert run(x=X + 8) == qd.QD_EALIGN
    assert run(x=WS + 1024) == qd.QD_EINVAL      # x inside the workspace
    layer = qd.Qwen3Layer(*[0x7f7000000000 + (i << 32) for i in range(13)])
    layer.k_cache = None
    assert run(model=_qwen3(layers=(qd.Qwen3Layer * 2)(layer, layer))) == qd.QD_EINVAL
    layer.k_cache = 0x7fd000000000 + 8
    assert run(model=_qwen3(layers=(qd.Qwen3Layer * 2)(layer, layer))) == qd.QD_EALIGN
    layer.k_cache = WS + 4096                    # a cache inside the workspace
    assert run(model=_qwen3(layers=(qd.Qwen3Layer * 2)(layer, layer))) == qd.QD_EINVAL
    layer.k_cache = layer.v_cache + 1024         # K and V caches overlapping
    assert run(model=_qwen3(layers=(qd.Qwen3Layer * 2)(layer, layer))) == qd.QD_EINVAL
    assert _call("qwen3_step_check", None, ctypes.byref(ctypes.c_uint32()), None) == qd.QD_EINVAL


def _gpu_visible():
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        n = ctypes.c_int(0)
        return hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0
    except OSError:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="fake pointers must never reach a real GPU")
def test_valid_args_reach_device_check():
    # with every argument valid, the only remaining failure on a host with no
    # GPU is the device check -- proving validation passed and nothing launched
    assert _call("qgemv_affine_i8_g64", A, 64, 1024, B, C, 1, None) == qd.QD_EDEVICE
    assert _call("qgemv_q4_0", A, 64, 512, B, C, 4, None) == qd.QD_EDEVICE
    assert _call("qd_stream_read", A, 1 << 20, B, None) == qd.QD_EDEVICE
    assert _call("qgemv_affine_i8_g64_f16", A, 64, 1024, B, C, 1, None) == qd.QD_EDEVICE
    lin = _lin((A, 0x7f3000000000, C, 64), (B, None, C + (1 << 20), 64))
    assert _call("qlinear_q4_0_gemv", lin, 2, 512, 0x7f4000000000, 4, 1, None) == qd.QD_EDEVICE
    assert _call("qlinear_q4_0_gemm", lin, 2, 512, 0x7f4000000000, 99, 0, None) == qd.QD_EDEVICE
    assert _call("affine_i8_g64_embed_rows", A, 64, 1024, _ids(0, 63), 2, C, 0,
                 None) == qd.QD_EDEVICE
    assert _call("qgemm_q4_0_prefill", A, 64, 512, B, C, 1500, None) == qd.QD_EDEVICE
    assert _call("q4_0_quantize", A, 3, 32, C, None) == qd.QD_EDEVICE
    assert _call("qgemv_affine_i8_g64_group", _affine_items((A, C, 64), (D, E, 32)), 2, 1024,
                 B, 4, None) == qd.QD_EDEVICE
    assert _call("qgemv_q4_0_group", _q4_items((A, C, 64), (D, E, 32)), 2, 512,
                 B, 4, None) == qd.QD_EDEVICE
    assert _call("affine_i8_g64_pack", A, B, C, 4, 64, A + (1 << 20), None) == qd.QD_EDEVICE
    ws = qd.attention_decode_workspace_bytes(16, 8, 128)
    assert _call("attention_decode", A, B, C, 16, 8, 128, 4096, 0, ctypes.c_float(0.088), 1,
                 OUT, WS, ws, None) == qd.QD_EDEVICE
    F = ctypes.c_float
    assert _call("rmsnorm_f16", A, B, C, 1024, F(1e-6), OUT, None) == qd.QD_EDEVICE
    assert _call("silu_mul_f16", A, B, A, 3072, None) == qd.QD_EDEVICE
    assert _call("qk_norm_rope_f16", A, B, C, OUT, OUT + 256, 16, 8, 128, F(1e-6), F(1e6), WS,
                 4096, 0x7f5000000000, 0x7f6000000000, WS + 64, None) == qd.QD_EDEVICE
    m = _qwen3()
    assert _call("qwen3_step_run", ctypes.byref(m), WS, qd.qwen3_step_workspace_bytes(m),
                 0x7fa000000000, 0x7fb000000000, None, 1, None) == qd.QD_EDEVICE


def _q4_ops(*specs):
    arr = (qd.Q40GemvOp * len(specs))()
    for i, sp in enumerate(specs):
        arr[i] = qd.Q40GemvOp(*sp)
    return arr


def test_errors_affine_step_rows():
    ops = (qd.AffineGemvOp * 1)(qd.AffineGemvOp(A, B, C, 64, 256, 0))
    wb = qd.lib().qgemv_affine_i8_g64_step_workspace_bytes
    plan = qd.StepPlan()
    for m in (0, 5):                     # 1..4 token rows
        assert wb(ops, 1, m) == 0
        assert _call("qgemv_affine_i8_g64_step_plan", ops, 1, m, WS, 1 << 20, ctypes.byref(plan),
                     None) == qd.QD_EINVAL
    p = qd.StepPlan(workspace=WS, nwg=256, lds_bytes=16384, n_ops=1, n_stages=1, m=5,
                    magic=0x51445354, tail=0, format=0)
    assert _call("qgemv_affine_i8_g64_step_run", ctypes.byref(p), None) == qd.QD_EINVAL
    if not _gpu_visible():
        for m in (1, 4):
            assert _call("qgemv_affine_i8_g64_step_plan", ops, 1, m, WS, 1 << 20,
                         ctypes.byref(plan), None) == qd.QD_EDEVICE


def test_errors_q4_0_step():
    wb = qd.lib().qgemv_q4_0_step_workspace_bytes
    ok = (A, B, C, 64, 256, 0)
    assert wb(None, 1, 1) == 0
    assert wb(_q4_ops((A, B, C, 64, 128, 0)), 1, 1) == 0       # cols % 256
    assert wb(_q4_ops(ok), 1, 2) == 0                          # m > 1
    f = "qgemv_q4_0_step_plan"
    plan = qd.StepPlan()
    P_ = ctypes.byref(plan)
    assert _call(f, None, 1, 1, WS, 1 << 20, P_, None) == qd.QD_EINVAL
    assert _call(f, _q4_ops(ok), 1, 1, None, 1 << 20, P_, None) == qd.QD_EINVAL
    assert _call(f, _q4_ops((A, B, C, 64, 128, 0)), 1, 1, WS, 1 << 20, P_, None) == qd.QD_ESHAPE
    assert _call(f, _q4_ops((A, B, C, 64, 8448, 0)), 1, 1, WS, 1 << 20, P_, None) == qd.QD_ESHAPE
    assert _call(f, _q4_ops((A, B, C + 2, 64, 256, 0)), 1, 1, WS, 1 << 20, P_, None) == qd.QD_EALIGN
    assert _call(f, _q4_ops((A, B + 4, C, 64, 256, 0)), 1, 1, WS, 1 << 20, P_, None) == qd.QD_EALIGN
    assert _call(f, _q4_ops((A, B, C, 64, 256, 1)), 1, 1, WS, 1 << 20, P_, None) == qd.QD_EINVAL
    assert _call(f, _q4_ops(ok, (D, B, E, 64, 512, 0)), 2, 1, WS, 1 << 20, P_,
                 None) == qd.QD_ESHAPE                         # one stage, two widths
    assert _call(f, _q4_ops(ok, (D, B, A + 64, 64, 256, 1)), 2, 1, WS, 1 << 20, P_,
                 None) == qd.QD_EINVAL                         # output over weights
    assert _call(f, _q4_ops(ok), 1, 1, WS + 16, 1 << 20, P_, None) == qd.QD_EALIGN
    assert _call(f, _q4_ops(ok), 1, 1, WS, 64, P_, None) == qd.QD_EINVAL
    # a plan of one format is refused by the other format's run and check
    for fmt, run, check in ((1, "qgemv_affine_i8_g64_step_run", "qgemv_affine_i8_g64_step_check"),
                            (0, "qgemv_q4_0_step_run", "qgemv_q4_0_step_check")):
        p = qd.StepPlan(workspace=WS, nwg=256, lds_bytes=16384, n_ops=1, n_stages=1, m=1,
                        magic=0x51445354, tail=0, format=fmt)
        assert _call(run, ctypes.byref(p), None) == qd.QD_EINVAL
        assert _call(check, ctypes.byref(p), ctypes.byref(ctypes.c_uint32()), None) == qd.QD_EINVAL
    # a Q4_0 plan never streams a last stage on its own
    p = qd.StepPlan(workspace=WS, nwg=256, lds_bytes=16384, n_ops=2, n_stages=2, m=1,
                    magic=0x51445354, tail=1, tail_w=A, tail_x=B, tail_y=C, tail_rows=64,
                    tail_cols=256, format=1)
    assert _call("qgemv_q4_0_step_run", ctypes.byref(p), None) == qd.QD_EINVAL
    if not _gpu_visible():
        assert _call(f, _q4_ops(ok), 1, 1, WS, 1 << 20, P_, None) == qd.QD_EDEVICE


def test_qwen3_step_workspace_offsets():
    # the scratch rows lie inside the workspace, 256-byte aligned, disjoint
    m = _qwen3()
    total = qd.qwen3_step_workspace_bytes(m)
    sizes = {"q": 4096, "k": 2048, "v": 2048, "attn": 4096, "opart": 8 * 1024 * 4,
             "gate": 6144, "up": 6144, "delta": 2048, "xalt": 2048, "qrope": 4096}
    spans = []
    for name, size in sizes.items():
        off = qd.qwen3_step_workspace_offset(m, name)
        assert off >= 256 and off % 256 == 0 and off + size <= total, name
        spans.append((off, off + size))
    spans.sort()
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    # with more than 8 K/V heads there are no partial rows
    m16 = _qwen3(heads=16, kv_heads=16, head_dim=64)
    assert qd.qwen3_step_workspace_offset(m16, "opart") == -1
    assert qd.qwen3_step_workspace_offset(m16, "attn") > 0
    assert qd.qwen3_step_workspace_offset(_qwen3(hidden=1000), "q") == -1
    assert qd.lib().qwen3_step_workspace_offset(ctypes.byref(m), 10) == -1
    assert qd.lib().qwen3_step_workspace_offset(None, 0) == -1


def test_errors_attention_decode_noalloc():
    # the same host-side checks as attention_decode (no workspace), and
    # QD_ESCRATCH for a head shape whose partials exceed the static scratch
    f = "attention_decode_noalloc"

    def call(q=A, k=B, v=C, heads=16, kvh=8, d=128, n=100, s=0, scale=0.088, f16=1, out=OUT):
        return _call(f, q, k, v, heads, kvh, d, n, s, ctypes.c_float(scale), f16, out, None)

    for bad in ({"q": None}, {"k": None}, {"v": None}, {"out": None}):
        assert call(**bad) == qd.QD_EINVAL
    assert call(f16=2) == qd.QD_EINVAL
    assert call(heads=24) == qd.QD_ESHAPE
    assert call(d=96) == qd.QD_ESHAPE
    assert call(n=0) == qd.QD_EINVAL
    assert call(s=100) == qd.QD_EINVAL
    assert call(scale=float("nan")) == qd.QD_EINVAL
    assert call(q=A + 8) == qd.QD_EALIGN
    assert call(out=B + 4096) == qd.QD_EINVAL         # output inside the K cache
    limit = 4 << 20
    assert qd.attention_decode_workspace_bytes(1024, 128, 128) <= limit
    if not _gpu_visible():  # fits: stops at the device check (a GPU would run it)
        assert call(heads=1024, kvh=128) == qd.QD_EDEVICE
    big = qd.attention_decode_workspace_bytes(8192, 1024, 128)
    assert big > limit
    assert call(heads=8192, kvh=1024) == qd.QD_ESCRATCH
    assert qd.attention_decode_workspace_bytes(32768, 4096, 64) > limit
    assert call(heads=32768, kvh=4096, d=64) == qd.QD_ESCRATCH
    assert qd.lib().qd_status_string(qd.QD_ESCRATCH).startswith(b"QD_ESCRATCH")
