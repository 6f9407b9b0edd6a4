"""GPU parity of the decoder-step ops and of the whole Qwen3 step.

turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step
with encode_rms_norm_bf16w(_perhead), encode_rope_neox_subdim,
encode_residual_add, encode_silu_mul and encode_attention_decode; f16
buffers, BF16 norm weights.

Ops: every stored f16 value must be the nearest-even rounding of the
oracle's exact value (f64) up to fp32 noise (1e-5 of max |out|), computed
from the kernel's own inputs.  The fused per-head norm + RoPE rounds the
normed head to f16 before rotating it (as the page stores it); where that
hidden intermediate lies within fp32 noise of a rounding tie, either
neighbour is a correct rounding, and the check takes the one the kernel's
output matches.

Whole step: the GPU step and the oracle's f16 step both round every buffer
to f16 but may take different sides of near-ties along the way, so their
difference is bounded by how far the f16 step itself sits from exact
arithmetic: normwise(gpu, oracle_f16) <= 2 * normwise(oracle_f16,
oracle_f64) + 2^-11, on the residual row, the new K/V cache rows and the
logits, position after position, eagerly and as a replayed HIP graph.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_transformer_decode_amd as qd
import synth
from helpers import DEV, check_f16_output, dev_f16, f16_rounding_interval, pack_on_device
from qwen3_models import empty_caches, oracle_model

pytestmark = pytest.mark.gpu

ULP16 = 2.0 ** -11


def _h(t):
    return t.float().cpu().numpy().astype(np.float64)


def _bits_f64(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _bf16_dev(bits):
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).to(DEV)


def _norm_w(n, key):
    w = synth.rng(30, key, n, 0).normal(1.0, 0.1, size=n).astype(np.float32)
    return synth.to_bf16_bits(w)


# ---- ops ----------------------------------------------------------------------

@pytest.mark.parametrize("n", [64, 1024, 2048, 8192])
@pytest.mark.parametrize("with_delta", [False, True])
def test_add_rmsnorm(n, with_delta):
    print(f"add_rmsnorm n={n} delta={with_delta}", flush=True)
    xb = synth.x_f16(1, n, key=(30, n, 1))[0]
    db = synth.x_f16(1, n, key=(30, n, 2))[0]
    wb = _norm_w(n, 3)
    x = dev_f16(xb)
    delta = dev_f16(db) if with_delta else None
    out = torch.full((n,), float("nan"), dtype=torch.float16, device=DEV)
    qd.rmsnorm_f16(x, delta, _bf16_dev(wb), n, 1e-6, out)
    torch.cuda.synchronize()
    x_new = _h(x)
    if with_delta:
        check_f16_output(x_new, _bits_f64(xb) + _bits_f64(db), "residual add")
    else:
        assert np.array_equal(x_new, _bits_f64(xb))
    ref = oracle.rms_norm(x_new, synth.bf16_bits_to_f32(wb).astype(np.float64),
                          float(np.float32(1e-6)))
    check_f16_output(_h(out), ref, "rmsnorm")


@pytest.mark.parametrize("n", [4, 3072, 6144, 100000])
def test_silu_mul(n):
    gb = synth.x_f16(1, n, key=(31, n, 1))[0]
    ub = synth.x_f16(1, n, key=(31, n, 2))[0]
    g, u = dev_f16(gb), dev_f16(ub)
    qd.silu_mul_f16(g, u, g, n)  # in place, as the page
    torch.cuda.synchronize()
    check_f16_output(_h(g), oracle.silu_mul(_bits_f64(gb), _bits_f64(ub)), f"silu_mul n={n}")


def _norm_rope_ref(x, w, eps, pos, theta, got):
    """Exact per-head norm -> f16 -> RoPE, taking, at each normed element
    within fp32 noise of an f16 rounding tie, the neighbour that the
    kernel's output matches best."""
    n_exact = oracle.rms_norm(x, w, eps)
    r = oracle.round_f16(n_exact)
    toward = np.where(n_exact > r, np.inf, -np.inf).astype(np.float16)
    alt = np.nextafter(r.astype(np.float16), toward).astype(np.float64)
    near = np.abs(n_exact - (r + alt) / 2) <= 1e-6 * np.abs(n_exact)
    d = x.shape[-1]
    half = d // 2
    ang = pos * np.power(float(theta), -2.0 * np.arange(half) / d)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = f16_rounding_interval(got)
    best = None
    for f1 in (False, True):
        for f2 in (False, True):
            n1 = np.where(f1 & near[..., :half], alt[..., :half], r[..., :half])
            n2 = np.where(f2 & near[..., half:], alt[..., half:], r[..., half:])
            y = np.concatenate([n1 * c - n2 * s, n2 * c + n1 * s], axis=-1)
            # distance of each candidate from the reals that round to `got`
            dist = np.maximum(0.0, np.maximum(lo - y, y - hi))
            err = np.maximum(dist[..., :half], dist[..., half:])
            if best is None:
                best, best_err = y, err
            else:
                take = np.concatenate([err < best_err, err < best_err], axis=-1)
                best = np.where(take, y, best)
                best_err = np.minimum(err, best_err)
    return best, int(near.sum())


@pytest.mark.parametrize("heads,kv,d,theta", [(16, 8, 128, 1e6), (4, 2, 64, 10000.0),
                                              (32, 8, 128, 1e6)])
@pytest.mark.parametrize("pos", [0, 1, 777, 40959])
def test_qk_norm_rope(heads, kv, d, theta, pos):
    print(f"qk_norm_rope heads={heads} kv={kv} d={d} pos={pos}", flush=True)
    cap = 40960
    qb = synth.x_f16(1, heads * d, key=(32, heads, 1))[0]
    kb = synth.x_f16(1, kv * d, key=(32, heads, 2))[0]
    vb = synth.x_f16(1, kv * d, key=(32, heads, 3))[0]
    qwb, kwb = _norm_w(d, 4), _norm_w(d, 5)
    q = dev_f16(qb)
    kc = torch.full((cap, kv, d), 7.0, dtype=torch.float16, device=DEV)
    vc = torch.full((cap, kv, d), 7.0, dtype=torch.float16, device=DEV)
    p = torch.tensor([pos], dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    eps = float(np.float32(1e-6))
    qd.qk_norm_rope_f16(q, dev_f16(kb), dev_f16(vb), _bf16_dev(qwb), _bf16_dev(kwb), heads, kv,
                        d, eps, theta, p, cap, kc, vc, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    wq = synth.bf16_bits_to_f32(qwb).astype(np.float64)
    wk = synth.bf16_bits_to_f32(kwb).astype(np.float64)
    gq = _h(q).reshape(heads, d)
    ref, _ = _norm_rope_ref(_bits_f64(qb).reshape(heads, d), wq, eps, pos,
                            float(np.float32(theta)), gq)
    check_f16_output(gq, ref, "q")
    gk = _h(kc[pos])
    ref, _ = _norm_rope_ref(_bits_f64(kb).reshape(kv, d), wk, eps, pos,
                            float(np.float32(theta)), gk)
    check_f16_output(gk, ref, "k row")
    assert np.array_equal(vc[pos].view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1), vb)
    # no other cache row was touched
    kc[pos] = 7.0
    vc[pos] = 7.0
    assert bool((kc == 7.0).all()) and bool((vc == 7.0).all())


def test_qk_norm_rope_position_outside_cache():
    heads, kv, d, cap = 16, 8, 128, 64
    qb = synth.x_f16(1, heads * d, key=(33, 0, 1))[0]
    q = dev_f16(qb)
    k = dev_f16(synth.x_f16(1, kv * d, key=(33, 0, 2))[0])
    w = _bf16_dev(_norm_w(d, 6))
    kc = torch.zeros((cap + 1, kv, d), dtype=torch.float16, device=DEV)
    vc = torch.zeros((cap + 1, kv, d), dtype=torch.float16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    for bad in (cap, -1):
        p = torch.tensor([bad], dtype=torch.int32, device=DEV)
        qd.qk_norm_rope_f16(q, k, k, w, w, heads, kv, d, 1e-6, 1e6, p, cap, kc, vc, err)
        torch.cuda.synchronize()
        assert int(err.item()) == 1
        err.zero_()
    assert not bool(kc.any()) and not bool(vc.any())
    assert np.array_equal(q.view(torch.int16).cpu().numpy().view(np.uint16), qb)


# ---- whole step ---------------------------------------------------------------

class GpuModel:
    """A synthetic Qwen3 on the device (packed by the library) + its oracle form."""

    def __init__(self, spec, capacity, layers=None):
        m = synth.qwen3_model(spec, layers=layers)
        self.spec, self.cap = spec, capacity
        self.om = oracle_model(spec, m)
        self.nl = len(m["layers"])
        self.keep = []
        dev_layers = []
        for L in m["layers"]:
            d = {name: pack_on_device(L[name]) for name in ("q", "k", "v", "o", "gate", "up",
                                                            "down")}
            d.update({name: _bf16_dev(L[name]) for name in ("in_norm", "q_norm", "k_norm",
                                                            "post_norm")})
            shape = (capacity, spec.kv_heads, spec.head_dim)
            d["k_cache"] = torch.zeros(shape, dtype=torch.float16, device=DEV)
            d["v_cache"] = torch.zeros(shape, dtype=torch.float16, device=DEV)
            dev_layers.append(d)
        self.layers = dev_layers
        self.final_norm = _bf16_dev(m["final_norm"])
        self.embed = pack_on_device(m["embed"])
        self.model = qd.qwen3_model(spec.hidden, spec.heads, spec.kv_heads, spec.head_dim,
                                    spec.inter, spec.vocab, capacity,
                                    float(np.float32(spec.eps)), float(np.float32(spec.theta)),
                                    dev_layers, self.final_norm, self.embed)
        self.wsb = qd.qwen3_step_workspace_bytes(self.model)
        assert self.wsb > 0
        self.ws = torch.zeros(self.wsb, dtype=torch.uint8, device=DEV)


def _bound(gpu, o16, o64):
    return 2 * oracle.normwise_error(o16, o64) + ULP16


def _check_step(gm, pos, x_gpu, logits_gpu, o16, o64, logit_rows=None):
    (x16, l16, k16, v16), (x64, l64, k64, v64) = o16, o64
    what = f"{gm.spec.name} pos={pos}"
    e = oracle.normwise_error(x_gpu, x16)
    assert e <= _bound(x_gpu, x16, x64), f"{what}: x {e:.3e} > {_bound(x_gpu, x16, x64):.3e}"
    lg = logits_gpu if logit_rows is None else logits_gpu[logit_rows]
    e = oracle.normwise_error(lg, l16)
    assert e <= _bound(lg, l16, l64), f"{what}: logits {e:.3e} > {_bound(lg, l16, l64):.3e}"
    for li in range(gm.nl):
        for name, ref16, ref64 in (("k", k16, k64), ("v", v16, v64)):
            got = _h(gm.layers[li][name + "_cache"][pos])
            b = _bound(got, ref16[li][pos], ref64[li][pos])
            e = oracle.normwise_error(got, ref16[li][pos])
            assert e <= b, f"{what}: layer {li} {name} row {e:.3e} > {b:.3e}"


def _oracle_runs(gm, xs, logit_rows=None):
    """The oracle's f16 and exact steps over the rows xs at positions 0, 1, ..."""
    spec = gm.spec
    k16, v16 = empty_caches(spec, gm.cap, gm.nl)
    k64, v64 = empty_caches(spec, gm.cap, gm.nl)
    out = []
    for pos, x in enumerate(xs):
        x16, l16 = oracle.qwen3_step(x, pos, gm.om, k16, v16, f16=True, logit_rows=logit_rows)
        x64, l64 = oracle.qwen3_step(x, pos, gm.om, k64, v64, f16=False, logit_rows=logit_rows)
        out.append(((x16, l16, k16, v16), (x64, l64, k64, v64)))
    return out


def test_step_tiny_eager_and_graph_replay():
    spec = synth.QWEN3_TINY_STEP
    gm = GpuModel(spec, capacity=16)
    steps = 9
    xs_bits = synth.x_f16(steps, spec.hidden, key=(34, 0, 0))
    xs = [_bits_f64(b) for b in xs_bits]
    ref = _oracle_runs(gm, xs)
    pos = torch.zeros(1, dtype=torch.int32, device=DEV)
    x = torch.empty(spec.hidden, dtype=torch.float16, device=DEV)
    logits = torch.empty(spec.vocab, dtype=torch.float16, device=DEV)

    def step():
        qd.qwen3_step_run(gm.model, gm.ws, gm.wsb, x, pos, logits, advance=True)

    # eager steps 0..2
    for p in range(3):
        x.copy_(dev_f16(xs_bits[p]))
        step()
        torch.cuda.synchronize()
        assert int(pos.item()) == p + 1
        _check_step(gm, p, _h(x), _h(logits), *ref[p])
    # the same step captured once and replayed for positions 3..8
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    x_in = torch.empty_like(x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            x.copy_(x_in)
            step()
    torch.cuda.synchronize()
    assert int(pos.item()) == 3        # capture ran nothing
    for p in range(3, steps):
        x_in.copy_(dev_f16(xs_bits[p]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(pos.item()) == p + 1
        _check_step(gm, p, _h(x), _h(logits), *ref[p])
    assert qd.qwen3_step_check(gm.ws) == 0


def test_step_replay_matches_eager_bit_for_bit():
    spec = synth.QWEN3_TINY_STEP
    outs = []
    for use_graph in (False, True):
        gm = GpuModel(spec, capacity=8)
        pos = torch.zeros(1, dtype=torch.int32, device=DEV)
        x = torch.empty(spec.hidden, dtype=torch.float16, device=DEV)
        logits = torch.empty(spec.vocab, dtype=torch.float16, device=DEV)
        xs_bits = synth.x_f16(6, spec.hidden, key=(35, 0, 0))
        x_in = torch.empty_like(x)

        def step():
            x.copy_(x_in)
            qd.qwen3_step_run(gm.model, gm.ws, gm.wsb, x, pos, logits, advance=True)

        if use_graph:
            s = torch.cuda.Stream()
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    step()
            run = g.replay
        else:
            run = step
        rec = []
        for p in range(6):
            x_in.copy_(dev_f16(xs_bits[p]))
            torch.cuda.synchronize()
            run()
            torch.cuda.synchronize()
            rec.append((x.clone(), logits.clone(), gm.layers[1]["k_cache"][p].clone()))
        outs.append(rec)
    for (xa, la, ka), (xb, lb, kb) in zip(*outs):
        assert torch.equal(xa.view(torch.int16), xb.view(torch.int16))
        assert torch.equal(la.view(torch.int16), lb.view(torch.int16))
        assert torch.equal(ka.view(torch.int16), kb.view(torch.int16))


def test_step_position_outside_cache_is_flagged():
    spec = synth.QWEN3_TINY_STEP
    gm = GpuModel(spec, capacity=4)
    pos = torch.tensor([4], dtype=torch.int32, device=DEV)
    x = dev_f16(synth.x_f16(1, spec.hidden, key=(36, 0, 0))[0])
    qd.qwen3_step_run(gm.model, gm.ws, gm.wsb, x, pos, None, advance=False)
    assert qd.qwen3_step_check(gm.ws) == 1
    assert qd.qwen3_step_check(gm.ws) == 0   # cleared
    for L in gm.layers:
        assert not bool(L["k_cache"].any()) and not bool(L["v_cache"].any())


def test_step_qwen3_0_6b_shape_two_layers():
    # the real widths (1024 hidden, 16/8 heads of 128, 3072 inter, 151936
    # vocab) over two layers, logits sampled for the oracle
    spec = synth.QWEN3_0_6B_STEP
    gm = GpuModel(spec, capacity=8, layers=2)
    rows = np.unique(np.concatenate([np.random.default_rng(7).integers(0, spec.vocab, 512),
                                     [0, spec.vocab - 1]]))
    xs_bits = synth.x_f16(3, spec.hidden, key=(37, 0, 0))
    ref = _oracle_runs(gm, [_bits_f64(b) for b in xs_bits], logit_rows=rows)
    pos = torch.zeros(1, dtype=torch.int32, device=DEV)
    x = torch.empty(spec.hidden, dtype=torch.float16, device=DEV)
    logits = torch.empty(spec.vocab, dtype=torch.float16, device=DEV)
    for p in range(3):
        print(f"qwen3-0.6b 2-layer step pos={p}", flush=True)
        x.copy_(dev_f16(xs_bits[p]))
        qd.qwen3_step_run(gm.model, gm.ws, gm.wsb, x, pos, logits, advance=True)
        torch.cuda.synchronize()
        _check_step(gm, p, _h(x), _h(logits), *ref[p], logit_rows=rows)


def test_step_without_logits_odd_layers_advancing():
    # three layers (an odd count), no LM head: the last residual add runs as
    # its own kernel, which also advances the position
    spec = synth.QWEN3_TINY_STEP
    gm = GpuModel(spec, capacity=8, layers=3)
    xs_bits = synth.x_f16(4, spec.hidden, key=(38, 0, 0))
    k16, v16 = empty_caches(spec, gm.cap, gm.nl)
    k64, v64 = empty_caches(spec, gm.cap, gm.nl)
    om = dict(gm.om, embed=None)
    pos = torch.zeros(1, dtype=torch.int32, device=DEV)
    x = torch.empty(spec.hidden, dtype=torch.float16, device=DEV)
    for p in range(4):
        x.copy_(dev_f16(xs_bits[p]))
        qd.qwen3_step_run(gm.model, gm.ws, gm.wsb, x, pos, None, advance=True)
        torch.cuda.synchronize()
        assert int(pos.item()) == p + 1
        xr = _bits_f64(xs_bits[p])
        x16, _ = oracle.qwen3_step(xr, p, om, k16, v16, f16=True)
        x64, _ = oracle.qwen3_step(xr, p, om, k64, v64, f16=False)
        got = _h(x)
        e = oracle.normwise_error(got, x16)
        assert e <= _bound(got, x16, x64), f"pos={p}: x {e:.3e}"
        for li in range(3):
            got_k = _h(gm.layers[li]["k_cache"][p])
            assert oracle.normwise_error(got_k, k16[li][p]) <= _bound(got_k, k16[li][p],
                                                                      k64[li][p])
    assert qd.qwen3_step_check(gm.ws) == 0


@pytest.mark.parametrize("heads,kv_heads,head_dim", [(4, 4, 64), (8, 2, 64), (16, 2, 128),
                                                     (8, 1, 128), (16, 16, 64)])
def test_step_head_groupings(heads, kv_heads, head_dim):
    # 1, 4 and 8 query heads per K/V head (the fused attention prologue's
    # other instances; 16 K/V heads take the o projection as its own GEMV
    # after the combine), one layer, positions 0..69: with a 4096-row cache the
    # attention chunks hold 32 (d 128) or 64 (d 64) rows, so the window
    # crosses chunk boundaries and the appended row moves between chunks
    spec = synth.Qwen3Spec(f"qwen3-g{heads // kv_heads}-d{head_dim}", 256, heads, kv_heads,
                           head_dim, 512, 1000, 1)
    print(f"step heads={heads} kv={kv_heads} d={head_dim}", flush=True)
    gm = GpuModel(spec, capacity=4096)
    positions = list(range(70))
    xs_bits = synth.x_f16(len(positions), spec.hidden, key=(39, heads, head_dim))
    ref = _oracle_runs(gm, [_bits_f64(b) for b in xs_bits])
    pos = torch.zeros(1, dtype=torch.int32, device=DEV)
    x = torch.empty(spec.hidden, dtype=torch.float16, device=DEV)
    logits = torch.empty(spec.vocab, dtype=torch.float16, device=DEV)
    for p in positions:
        x.copy_(dev_f16(xs_bits[p]))
        qd.qwen3_step_run(gm.model, gm.ws, gm.wsb, x, pos, logits, advance=True)
        torch.cuda.synchronize()
        _check_step(gm, p, _h(x), _h(logits), *ref[p])
    assert qd.qwen3_step_check(gm.ws) == 0
