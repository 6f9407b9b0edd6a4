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


# ---- the f16 buffer model, pinned by the page's own buffer list -------------
#
# turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs -- `Work` and
# `ensure_work` allocate every activation buffer of the step (x, normed, q,
# attn, delta, gate, up, logits and the per-layer K/V caches) as 16-bit words;
# `Qwen3AsrMetalEngine::step` encodes one kernel per op, each reading and
# writing those buffers (the per-head norms, the RoPE and the SiLU-mul in
# place).  The machine below executes that encoder list literally on
# numpy float16 arrays: whatever an encoder writes is stored in a 16-bit
# buffer, so the rounding points follow from the buffers' type, not from a
# list of roundings.  Each encoder's arithmetic is the exact (f64) value of
# its inputs (the page does not give kernel internals).  The oracle's f16
# step must match it bit for bit.

class _PageBuffers:
    """The step's scratch as the page allocates it: f16 words."""

    def __init__(self, spec, capacity, n_layers):
        hid, qw, kw = spec.hidden, spec.heads * spec.head_dim, spec.kv_heads * spec.head_dim
        h = lambda n: np.zeros(n, dtype=np.float16)
        self.x, self.normed, self.q, self.attn = h(hid), h(hid), h(qw), h(qw)
        self.delta, self.gate, self.up = h(hid), h(spec.inter), h(spec.inter)
        self.logits = h(spec.vocab)
        self.k = [np.zeros((capacity, kw), dtype=np.float16) for _ in range(n_layers)]
        self.v = [np.zeros((capacity, kw), dtype=np.float16) for _ in range(n_layers)]


class _PageMachine:
    """Encoders of the step on f16 buffers; arithmetic in f64 from the
    buffers' values; a store into a buffer is a store into float16."""

    def __init__(self, spec, om, capacity):
        self.spec, self.om = spec, om
        self.dense = {}
        self.buf = _PageBuffers(spec, capacity, len(om["layers"]))

    def _w(self, blob, rows, cols):
        key = id(blob)
        if key not in self.dense:
            self.dense[key] = reference_np.affine_dense(blob, rows, cols)
        return self.dense[key]

    # encode_dequant_int8_gemv_resident: y = W x
    def gemv(self, blob, rows, cols, src, dst):
        dst[...] = self._w(blob, rows, cols) @ src.astype(np.float64)

    # encode_rms_norm_bf16w(_perhead): per row of `width` elements
    def rms_norm(self, src, w, dst, width):
        a = src.astype(np.float64).reshape(-1, width)
        inv = 1.0 / np.sqrt((a * a).sum(axis=1, keepdims=True) / width + self.om["eps"])
        dst[...] = (a * inv * np.asarray(w)[None, :]).reshape(dst.shape)

    # encode_rope_neox_subdim with rotary width = head_dim, in place
    def rope(self, buf, position, heads):
        d = self.spec.head_dim
        a = buf.astype(np.float64).reshape(heads, d)
        i = np.arange(d // 2, dtype=np.float64)
        z = (a[:, : d // 2] + 1j * a[:, d // 2:]) * np.exp(
            1j * position * self.om["theta"] ** (-2.0 * i / d))
        buf[...] = np.concatenate([z.real, z.imag], axis=1).reshape(-1)

    # encode_attention_decode over rows [0, position]
    def attention(self, layer, position):
        s = self.spec
        grp = s.heads // s.kv_heads
        scale = float(np.float32(1.0) / np.sqrt(np.float32(s.head_dim)))
        q = self.buf.q.astype(np.float64).reshape(s.heads, s.head_dim)
        K = self.buf.k[layer][: position + 1].astype(np.float64).reshape(-1, s.kv_heads,
                                                                          s.head_dim)
        V = self.buf.v[layer][: position + 1].astype(np.float64).reshape(-1, s.kv_heads,
                                                                          s.head_dim)
        out = np.empty((s.heads, s.head_dim))
        for h in range(s.heads):
            sc = K[:, h // grp, :] @ q[h] * scale
            e = np.exp(sc - sc.max())
            out[h] = (e / e.sum()) @ V[:, h // grp, :]
        self.buf.attn[...] = out.reshape(-1)

    def step(self, row, position, logit_rows):
        s, om, b = self.spec, self.om, self.buf
        hid, H, KV, d, inter = s.hidden, s.heads, s.kv_heads, s.head_dim, s.inter
        b.x[...] = row                                   # write_buffer_bytes(x, row)
        for li, L in enumerate(om["layers"]):
            kr, vr = b.k[li][position], b.v[li][position]  # (cache, kv_row)
            self.rms_norm(b.x, L["in_norm"], b.normed, hid)
            self.gemv(L["q"], H * d, hid, b.normed, b.q)
            self.gemv(L["k"], KV * d, hid, b.normed, kr)
            self.gemv(L["v"], KV * d, hid, b.normed, vr)
            self.rms_norm(b.q, L["q_norm"], b.q, d)
            self.rms_norm(kr, L["k_norm"], kr, d)
            self.rope(b.q, position, H)
            self.rope(kr, position, KV)
            self.attention(li, position)
            self.gemv(L["o"], hid, H * d, b.attn, b.delta)
            b.x[...] = b.x.astype(np.float64) + b.delta   # encode_residual_add
            self.rms_norm(b.x, L["post_norm"], b.normed, hid)
            self.gemv(L["gate"], inter, hid, b.normed, b.gate)
            self.gemv(L["up"], inter, hid, b.normed, b.up)
            g, u = b.gate.astype(np.float64), b.up.astype(np.float64)
            b.gate[...] = g / (1.0 + np.exp(-g)) * u      # encode_silu_mul, in place
            self.gemv(L["down"], hid, inter, b.gate, b.delta)
            b.x[...] = b.x.astype(np.float64) + b.delta
        self.rms_norm(b.x, om["final_norm"], b.normed, hid)
        self.gemv(om["embed"], s.vocab, hid, b.normed, b.logits)
        lg = b.logits.astype(np.float64)
        return b.x.astype(np.float64), lg if logit_rows is None else lg[logit_rows]


def _machine_vs_step(step_fn, spec, om, rows, positions):
    """Run the page machine and `step_fn` (the oracle's qwen3_step or a
    mutant of it) over the same rows; True when every stored value agrees
    bit for bit (residual row, logits, every layer's new K/V rows)."""
    cap = max(positions) + 1
    pm = _PageMachine(spec, om, cap)
    kc, vc = empty_caches(spec, cap, len(om["layers"]))
    sel = np.arange(0, spec.vocab, 7)
    for row, pos in zip(rows, positions):
        mx, ml = pm.step(row, pos, sel)
        ox, ol = step_fn(row, pos, om, kc, vc, f16=True, logit_rows=sel)
        same = np.array_equal(mx, ox) and np.array_equal(ml, ol)
        for li in range(len(om["layers"])):
            same &= np.array_equal(pm.buf.k[li][pos].astype(np.float64), kc[li][pos].reshape(-1))
            same &= np.array_equal(pm.buf.v[li][pos].astype(np.float64), vc[li][pos].reshape(-1))
        if not same:
            return False
    return True


def _pin_inputs():
    spec = synth.QWEN3_TINY_STEP
    om = oracle_model(spec, synth.qwen3_model(spec))
    # rows that are not f16 numbers, so the store into x itself rounds; the
    # third position is far from 0 so the RoPE angles are large
    rows = np.random.default_rng(6).standard_normal((3, spec.hidden)) * 0.5
    return spec, om, rows, [0, 1, 3]


def test_f16_step_equals_the_page_buffer_machine():
    spec, om, rows, positions = _pin_inputs()
    assert _machine_vs_step(oracle.qwen3_step, spec, om, rows, positions)


def _rounding_mutants():
    """Variants of oracle.qwen3_step with one of its f16 roundings dropped or
    done in BF16 instead, built from its source (the mistakes a reading of
    the page's buffers could make)."""
    import ast
    import inspect
    import textwrap

    src = textwrap.dedent(inspect.getsource(oracle.qwen3_step))
    tree = ast.parse(src)
    sites = [n for n in ast.walk(tree)
             if isinstance(n, ast.Call) and isinstance(n.func, ast.Name) and n.func.id == "r"]
    assert len(sites) >= 15, len(sites)

    def bf16(v):
        return synth.bf16_bits_to_f32(synth.to_bf16_bits(
            np.asarray(v, dtype=np.float64).astype(np.float32))).astype(np.float64)

    for i in range(len(sites)):
        for kind in ("drop", "bf16"):
            t = ast.parse(src)
            calls = [n for n in ast.walk(t) if isinstance(n, ast.Call) and
                     isinstance(n.func, ast.Name) and n.func.id == "r"]
            c = calls[i]
            what = f"{kind} r() at line {c.lineno}: {ast.unparse(c)[:60]}"

            class Swap(ast.NodeTransformer):
                def visit_Call(self, node):
                    self.generic_visit(node)
                    if node is c:
                        if kind == "drop":
                            return node.args[0]
                        return ast.Call(func=ast.Name("_round_bf16", ast.Load()),
                                        args=node.args, keywords=[])
                    return node

            t = ast.fix_missing_locations(Swap().visit(t))
            ns = dict(vars(oracle))
            ns["_round_bf16"] = bf16
            exec(compile(t, "<mutant>", "exec"), ns)
            yield what, ns["qwen3_step"]


def _caught(fn, spec, om, rows, positions):
    """A mutant is caught when the pin sees a difference, or when it stops
    with an error (a GEMV of the f16 step refuses inputs that are not f16
    numbers: a dropped rounding in front of it cannot pass unnoticed)."""
    try:
        return not _machine_vs_step(fn, spec, om, rows, positions)
    except AssertionError:
        return True


def test_buffer_machine_pin_catches_every_rounding_mutant():
    # every stored-buffer rounding of the oracle matters to the pin: dropping
    # any one of them, or doing it in BF16, breaks bit equality with the
    # page machine
    spec, om, rows, positions = _pin_inputs()
    survivors = [what for what, fn in _rounding_mutants()
                 if not _caught(fn, spec, om, rows, positions)]
    assert not survivors, survivors


def _step_with(**replace):
    import inspect
    import textwrap
    ns = dict(vars(oracle))
    ns.update(replace)
    exec(compile(textwrap.dedent(inspect.getsource(oracle.qwen3_step)), "<mutant>", "exec"), ns)
    return ns["qwen3_step"]


def test_buffer_machine_pin_catches_an_extra_rounding():
    # roundings where the page stores nothing must break the pin too: the
    # attention's scores kept in f16, or the norm's mean square reduced in f16
    spec, om, rows, positions = _pin_inputs()

    def attention_f16_scores(q, k, v, length, scale, kv_start=0):
        group = q.shape[0] // k.shape[1]
        out = np.empty_like(q)
        for h in range(q.shape[0]):
            s = oracle.round_f16(scale * (k[kv_start:length, h // group, :] @ q[h]))
            p = np.exp(s - s.max())
            out[h] = (p / p.sum()) @ v[kv_start:length, h // group, :]
        return out

    def rms_norm_f16_mean(x, w, eps):
        x = np.asarray(x, dtype=np.float64)
        ms = oracle.round_f16(np.mean(x * x, axis=-1, keepdims=True))
        return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)

    assert _caught(_step_with(attention_decode=attention_f16_scores), spec, om, rows, positions)
    assert _caught(_step_with(rms_norm=rms_norm_f16_mean), spec, om, rows, positions)
    # and the unmutated copy built the same way still passes
    assert not _caught(_step_with(), spec, om, rows, positions)
