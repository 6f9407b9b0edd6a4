"""GPU parity of the fused Qwen3 decode step where it runs for real: long
caches, large positions, full depth, and op by op inside one step.

turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step
(encode_rope_neox_subdim at `position`; the K/V caches sized by
`ensure_work`'s capacity; attention over rows [0, position]).

Caches are pre-filled with seeded f16 rows on the device, and the oracle starts
from the device's cache rows [0, p), so a step at position p attends p + 1 rows without p
earlier steps.  Two kinds of check:

* Whole step: as in test_gpu_decoder_step -- normwise(GPU, oracle f16) <=
  2 * normwise(oracle f16, oracle exact) + 2^-11 on the residual row, the
  new K/V rows and the logits.
* Op by op, from the rows the step stores (qwen3_step_workspace_offset),
  each op's output against the exact value of the same op applied to the
  GPU's own stored inputs:
    - q, k, v GEMVs (input RMSNorm built in LDS, never stored), gate, up
      (post-attention RMSNorm) and down (f16(silu(gate) * up)): each f16
      value the nearest-even rounding of the exact value within 1e-5 of
      max |out|, plus, per output, the effect of the hidden input's entries
      that lie within fp32 noise of an f16 tie rounding the other way;
    - the rotated q row and the appended K row: norm -> f16 -> RoPE -> f16
      of the GPU's q / k rows (tie-aware); the appended V row equals the
      GPU's v row bit for bit;
    - the attention row from the stored rotated q over the device's cache
      rows [0, p]: nearest-even within 1e-5;
    - the o projection's fp32 partial rows (one per K/V head, fused with the
      chunk merge): W_o over that head's columns times the stored attention
      row, normwise within 1e-5;
    - the residual row after attention, f16(x + f16(sum of the partial rows
      in head order, fp32)), and the final one, f16(x + down): bit for bit;
    - the logits (final norm staged in the LM head, sampled rows) as the
      GEMVs above.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_transformer_decode_amd as qd
import synth
from helpers import DEV, check_f16_output, dev_f16, near_tie_allowance, near_ties
from oracle import reference_np
from qwen3_models import empty_caches
from test_gpu_decoder_step import GpuModel, _bits_f64, _check_step, _h, _norm_rope_ref

pytestmark = pytest.mark.gpu

SPEC = synth.QWEN3_0_6B_STEP


def _prefill(gm, rows, key):
    """Fill cache rows [0, rows) of every layer with seeded f16 N(0, 1) rows
    on the device; returns the host bits per layer ((K, V) uint16 [rows, kv_w])."""
    kw = gm.spec.kv_heads * gm.spec.head_dim
    out = []
    for li, L in enumerate(gm.layers):
        kb = synth.x_f16(rows, kw, key=(60, key, 2 * li))
        vb = synth.x_f16(rows, kw, key=(60, key, 2 * li + 1))
        L["k_cache"][:rows].view(torch.int16).copy_(
            torch.from_numpy(kb.view(np.int16).reshape(rows, gm.spec.kv_heads, -1)))
        L["v_cache"][:rows].view(torch.int16).copy_(
            torch.from_numpy(vb.view(np.int16).reshape(rows, gm.spec.kv_heads, -1)))
        out.append((kb, vb))
    torch.cuda.synchronize()
    return out


def _oracle_step(gm, pos, x_row, logit_rows):
    """The oracle's f16 and exact steps at `pos`, its caches holding the
    device's cache rows [0, pos) (pre-filled, or written by earlier steps;
    a step writes only row pos)."""
    spec = gm.spec
    dev_rows = [(_h(L["k_cache"][:pos]), _h(L["v_cache"][:pos])) for L in gm.layers]
    res = []
    for f16 in (True, False):
        kc, vc = empty_caches(spec, pos + 1, gm.nl)
        for li, (kr, vr) in enumerate(dev_rows):
            kc[li][:pos] = kr
            vc[li][:pos] = vr
        x, lg = oracle.qwen3_step(x_row, pos, gm.om, kc, vc, f16=f16, logit_rows=logit_rows)
        res.append((x, lg, kc, vc))
    return res


def _ws_f16(gm, name, n):
    off = qd.qwen3_step_workspace_offset(gm.model, name)
    assert off >= 0, name
    return _h(gm.ws[off:off + 2 * n].view(torch.float16))


def _ws_f32(gm, name, n):
    off = qd.qwen3_step_workspace_offset(gm.model, name)
    assert off >= 0, name
    return gm.ws[off:off + 4 * n].view(torch.float32).cpu().numpy()


def _gemv_hidden_input(got, blob, rows, cols, x_exact, what, row_sel=None, rel=2e-6):
    """A GEMV whose input row the kernel builds and rounds to f16 in LDS
    (never stored): each output must be the nearest-even rounding of W r
    (r = the f16 rounding of the exact input) within 1e-5 of max |out|, plus,
    per output, what the input entries lying within fp32 noise (rel) of an
    f16 tie could add by rounding the other way."""
    r, alt, near = near_ties(x_exact, rel)
    ref = oracle.affine_gemv_f64(blob, rows, cols, r, row_sel=row_sel)
    allow = None
    if near.any():
        wc = reference_np.affine_dense_sub(blob, rows, cols, row_sel, np.nonzero(near)[0])
        allow = near_tie_allowance(wc, r, alt, near)
    check_f16_output(got, ref, what, allowance=allow)


def _op_checks(gm, x0, pos, x_gpu, logits_gpu, logit_rows):
    """The op-by-op checks of one step of a one-layer model (module doc)."""
    s, om = gm.spec, gm.om
    L = om["layers"][0]
    hid, H, KV, d, inter = s.hidden, s.heads, s.kv_heads, s.head_dim, s.inter
    eps, theta = om["eps"], om["theta"]
    what = f"pos={pos}"
    gl = gm.layers[0]
    # q, k, v with the input norm staged
    n1 = oracle.rms_norm(x0, L["in_norm"], eps)
    q = _ws_f16(gm, "q", H * d)
    k = _ws_f16(gm, "k", KV * d)
    v = _ws_f16(gm, "v", KV * d)
    _gemv_hidden_input(q, L["q"], H * d, hid, n1, f"{what} q")
    _gemv_hidden_input(k, L["k"], KV * d, hid, n1, f"{what} k")
    _gemv_hidden_input(v, L["v"], KV * d, hid, n1, f"{what} v")
    # per-head norm + RoPE of q (stored row) and of k (the appended cache row)
    qr = _ws_f16(gm, "qrope", H * d).reshape(H, d)
    ref, _ = _norm_rope_ref(q.reshape(H, d), L["q_norm"], eps, pos, theta, qr)
    check_f16_output(qr, ref, f"{what} rotated q")
    krow = _h(gl["k_cache"][pos]).reshape(KV, d)
    ref, _ = _norm_rope_ref(k.reshape(KV, d), L["k_norm"], eps, pos, theta, krow)
    check_f16_output(krow, ref, f"{what} appended K row")
    assert np.array_equal(_h(gl["v_cache"][pos]).reshape(-1), v), f"{what} appended V row"
    # attention over rows [0, pos] of the device's caches from the stored q
    kc = _h(gl["k_cache"][:pos + 1])
    vc = _h(gl["v_cache"][:pos + 1])
    scale = float(np.float32(1.0) / np.sqrt(np.float32(d)))
    attn = _ws_f16(gm, "attn", H * d)
    check_f16_output(attn, oracle.attention_decode(qr, kc, vc, pos + 1, scale).reshape(-1),
                     f"{what} attention")
    # the o projection inside the merge: fp32 partial rows per K/V head over
    # that head's columns of the stored attention row
    wo = reference_np.affine_dense(L["o"], hid, H * d)
    gw = (H // KV) * d
    opart_ref = np.stack([wo[:, j * gw:(j + 1) * gw] @ attn[j * gw:(j + 1) * gw]
                          for j in range(KV)])
    opart = _ws_f32(gm, "opart", KV * hid).reshape(KV, hid)
    e = oracle.normwise_error(opart, opart_ref)
    assert e <= 1e-5, f"{what}: o partial rows {e:.3e}"
    # residual after attention: f16(x + f16(partials summed in head order, fp32))
    acc = opart[0].astype(np.float32)
    for j in range(1, KV):
        acc = (acc + opart[j]).astype(np.float32)
    o16 = acc.astype(np.float16).astype(np.float32)
    xa_ref = (x0.astype(np.float32) + o16).astype(np.float16).astype(np.float64)
    xa = _ws_f16(gm, "xalt", hid)
    assert np.array_equal(xa, xa_ref), f"{what}: residual after attention"
    # gate, up with the post-attention norm staged; down with SiLU-mul staged
    n2 = oracle.rms_norm(xa, L["post_norm"], eps)
    gate = _ws_f16(gm, "gate", inter)
    up = _ws_f16(gm, "up", inter)
    _gemv_hidden_input(gate, L["gate"], inter, hid, n2, f"{what} gate")
    _gemv_hidden_input(up, L["up"], inter, hid, n2, f"{what} up")
    down = _ws_f16(gm, "delta", hid)
    _gemv_hidden_input(down, L["down"], hid, inter, oracle.silu_mul(gate, up), f"{what} down")
    # final residual row and the logits (final norm staged in the LM head)
    x_ref = (xa.astype(np.float32) + down.astype(np.float32)).astype(np.float16)
    assert np.array_equal(x_gpu, x_ref.astype(np.float64)), f"{what}: final residual row"
    _gemv_hidden_input(logits_gpu[logit_rows], om["embed"], s.vocab, hid,
                       oracle.rms_norm(x_gpu, om["final_norm"], eps), f"{what} logits",
                       row_sel=logit_rows)


def _logit_rows(spec, seed):
    return np.unique(np.concatenate([np.random.default_rng(seed).integers(0, spec.vocab, 256),
                                     [0, spec.vocab - 1]]))


def _run_positions(gm, positions, xs_bits, rows, graph_from=None):
    """Step at each position (eagerly, or from `graph_from` on by replaying
    one captured step that advances the position), checking every step op by
    op and against the oracle."""
    pos_t = torch.zeros(1, dtype=torch.int32, device=DEV)
    x = torch.empty(gm.spec.hidden, dtype=torch.float16, device=DEV)
    x_in = torch.empty_like(x)
    logits = torch.empty(gm.spec.vocab, dtype=torch.float16, device=DEV)
    graph = None
    for i, p in enumerate(positions):
        print(f"qwen3-0.6b 1-layer step pos={p} cap={gm.cap}", flush=True)
        x_in.copy_(dev_f16(xs_bits[i]))
        if graph_from is not None and i >= graph_from:
            if graph is None:
                pos_t.fill_(p)
                torch.cuda.synchronize()
                s = torch.cuda.Stream()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.stream(s):
                    with torch.cuda.graph(graph, stream=s):
                        x.copy_(x_in)
                        qd.qwen3_step_run(gm.model, gm.ws, gm.wsb, x, pos_t, logits,
                                          advance=True)
                torch.cuda.synchronize()
                assert int(pos_t.item()) == p  # capture ran nothing
            assert int(pos_t.item()) == p
            graph.replay()
        else:
            pos_t.fill_(p)
            x.copy_(x_in)
            qd.qwen3_step_run(gm.model, gm.ws, gm.wsb, x, pos_t, logits, advance=False)
        torch.cuda.synchronize()
        x0 = _bits_f64(xs_bits[i])
        xg, lg = _h(x), _h(logits)
        _op_checks(gm, x0, p, xg, lg, rows)
        o16, o64 = _oracle_step(gm, p, x0, rows)
        _check_step(gm, p, xg, lg, o16, o64, logit_rows=rows)
    assert qd.qwen3_step_check(gm.ws) == 0


def test_step_long_cache_positions_op_by_op():
    # positions on both sides of where the attention's chunk length starts
    # following 1.5 sqrt(rows) (~455 rows), and deep into a 4096-row cache:
    # the RoPE angles grow with the position and the window spans many chunks
    gm = GpuModel(SPEC, capacity=4096, layers=1)
    _prefill(gm, 4096, key=1)
    positions = [455, 456, 1023, 2047, 4095]
    xs = synth.x_f16(len(positions), SPEC.hidden, key=(61, 0, 0))
    _run_positions(gm, positions, xs, _logit_rows(SPEC, 1))


def test_step_position_40959_op_by_op():
    gm = GpuModel(SPEC, capacity=40960, layers=1)
    _prefill(gm, 40960, key=2)
    positions = [40959]
    xs = synth.x_f16(1, SPEC.hidden, key=(61, 1, 0))
    _run_positions(gm, positions, xs, _logit_rows(SPEC, 2))


def test_step_large_positions_graph_replay():
    # one captured step, replayed: it reads and advances the position on the
    # device (4093 eagerly, then 4094 and 4095 from the graph)
    gm = GpuModel(SPEC, capacity=4096, layers=1)
    _prefill(gm, 4096, key=3)
    positions = [4093, 4094, 4095]
    xs = synth.x_f16(len(positions), SPEC.hidden, key=(61, 2, 0))
    _run_positions(gm, positions, xs, _logit_rows(SPEC, 3), graph_from=1)


def test_step_qwen3_0_6b_all_28_layers():
    # the whole Qwen3-0.6B-shaped decoder (28 layers, the tied 151936-row
    # head, logits sampled) at two positions over 300 pre-filled cache rows:
    # one eager step, then one replayed graph
    gm = GpuModel(SPEC, capacity=512)
    assert gm.nl == 28
    _prefill(gm, 300, key=4)
    rows = _logit_rows(SPEC, 4)
    xs = synth.x_f16(2, SPEC.hidden, key=(61, 3, 0))
    pos_t = torch.zeros(1, dtype=torch.int32, device=DEV)
    x = torch.empty(SPEC.hidden, dtype=torch.float16, device=DEV)
    x_in = torch.empty_like(x)
    logits = torch.empty(SPEC.vocab, dtype=torch.float16, device=DEV)

    def step():
        x.copy_(x_in)
        qd.qwen3_step_run(gm.model, gm.ws, gm.wsb, x, pos_t, logits, advance=True)

    pos_t.fill_(300)
    x_in.copy_(dev_f16(xs[0]))
    print("qwen3-0.6b 28-layer step pos=300 eager", flush=True)
    step()
    torch.cuda.synchronize()
    o16, o64 = _oracle_step(gm, 300, _bits_f64(xs[0]), rows)
    _check_step(gm, 300, _h(x), _h(logits), o16, o64, logit_rows=rows)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    assert int(pos_t.item()) == 301
    x_in.copy_(dev_f16(xs[1]))
    print("qwen3-0.6b 28-layer step pos=301 graph", flush=True)
    g.replay()
    torch.cuda.synchronize()
    assert int(pos_t.item()) == 302
    o16, o64 = _oracle_step(gm, 301, _bits_f64(xs[1]), rows)
    _check_step(gm, 301, _h(x), _h(logits), o16, o64, logit_rows=rows)
    assert qd.qwen3_step_check(gm.ws) == 0
