"""GPU parity of the single-launch decode step over Q4_0 GEMVs
(qgemv_q4_0_step_*) against the oracle, GEMV by GEMV.

fuel-transformers 0.19.1, src/models/lazy_quantized_whisper.rs --
decoder_layer (q, k, v, then o, then fc1, then fc2, in decoder order) and
q_linear (the Q4_0 matmul of each projection).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_transformer_decode_amd as qd
import synth
from helpers import DEV, check_f32_output, dev_f32, dev_u8

pytestmark = pytest.mark.gpu


class Q4Step:
    def __init__(self, shapes, key, share_weights=None):
        """shapes: list of (rows, cols, stage).  share_weights: optional list
        giving, per op, the index of an earlier op whose weights it reuses
        (a full-depth decoder with one layer's matrices)."""
        self.shapes = shapes
        self.wq, self.wdev, self.xs, self.xdev, self.ys = [], [], [], [], []
        for i, (rows, cols, stage) in enumerate(shapes):
            j = share_weights[i] if share_weights is not None else i
            if j == i:
                w = synth.w_f32(rows, cols, key=(key, i, 0))
                self.wq.append(oracle.q4_0_quantize(w, rows, cols))
                self.wdev.append(dev_u8(self.wq[-1]))
            else:
                self.wq.append(self.wq[j])
                self.wdev.append(self.wdev[j])
            x = synth.x_f32(1, cols, key=(key, i, 1))
            self.xs.append(x)
            self.xdev.append(dev_f32(x))
            self.ys.append(torch.full((1, rows), float("nan"), dtype=torch.float32, device=DEV))
        self.ops = qd.make_q4_0_ops((w, x, y, r, c, s) for (r, c, s), w, x, y in
                                    zip(shapes, self.wdev, self.xdev, self.ys))
        nbytes = qd.qgemv_q4_0_step_workspace_bytes(self.ops, 1)
        assert nbytes > 0
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        self.plan = qd.qgemv_q4_0_step_plan(self.ops, 1, self.ws, nbytes)
        assert self.plan.format == 1 and self.plan.tail == 0

    def run(self):
        qd.qgemv_q4_0_step_run(self.plan)
        assert qd.qgemv_q4_0_step_check(self.plan) == 0

    def check(self, sample_rows=None, what=""):
        for i, (rows, cols, stage) in enumerate(self.shapes):
            sel = None
            if sample_rows and rows > sample_rows:
                sel = np.unique(np.concatenate([
                    np.random.default_rng(i).integers(0, rows, sample_rows), [0, rows - 1]]))
            ref = oracle.q4_0_gemm(self.wq[i], rows, cols, self.xs[i], row_sel=sel)
            got = self.ys[i].cpu().numpy()
            if sel is not None:
                got = got[:, sel]
            check_f32_output(got, ref, f"{what} op {i} ({rows}x{cols}, stage {stage})")


SMALL = [(130, 256, 0), (64, 256, 0), (17, 256, 0),    # three GEMVs sharing a stage
         (256, 512, 1),
         (3000, 256, 2), (3000, 256, 2),                 # more rows than waves
         (256, 4608, 3),                                 # several 64-block items per row
         (1, 256, 4),                                    # a single output
         (5000, 2304, 5)]                                # partial last item (72 blocks)


def test_q4_0_step_small_parity_and_relaunch():
    print("q4_0 step small", flush=True)
    st = Q4Step(SMALL, key=40)
    st.run()
    st.check(what="first launch")
    # a second launch with new inputs must read the new inputs
    for i, (rows, cols, stage) in enumerate(SMALL):
        x = synth.x_f32(1, cols, key=(41, i, 1))
        st.xs[i] = x
        st.xdev[i].copy_(dev_f32(x))
        st.ys[i].fill_(float("nan"))
    torch.cuda.synchronize()
    st.run()
    st.check(what="second launch")


def test_q4_0_step_graph_replays_bit_stable():
    print("q4_0 step graph", flush=True)
    st = Q4Step(SMALL[:6], key=42)
    st.run()
    first = [y.clone() for y in st.ys]
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            qd.qgemv_q4_0_step_run(st.plan)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in st.ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert qd.qgemv_q4_0_step_check(st.plan) == 0
        st.check(what=f"replay {rep}")
        # the walk and the summation order are fixed: every launch gives
        # the same bits
        for a, b in zip(first, st.ys):
            assert torch.equal(a, b)


def test_q4_0_step_whisper_large_full_depth_sampled():
    # the 192 Q4_0 GEMVs of a Whisper-large decoder step (32 layers, 128
    # stages), one layer's matrices shared by all layers, sampled rows
    print("q4_0 step whisper-large", flush=True)
    shapes, share = [], []
    layer = [(1280, 1280, 0), (1280, 1280, 0), (1280, 1280, 0), (1280, 1280, 1),
             (5120, 1280, 2), (1280, 5120, 3)]
    for l in range(synth.WHISPER_LARGE_LAYERS):
        for j, (r, c, s) in enumerate(layer):
            shapes.append((r, c, 4 * l + s))
            share.append(j)
    st = Q4Step(shapes, key=43, share_weights=share)
    assert st.plan.n_stages == 128
    for _ in range(3):
        st.run()
    st.check(sample_rows=32, what="whisper-large")


def test_q4_0_step_plan_rejects_bad_ops():
    t = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    base = t.data_ptr()
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=DEV)
    w, x, y = base, base + (1 << 20), base + (2 << 20)
    with pytest.raises(qd.QDError) as e:   # cols must be a multiple of 256
        qd.qgemv_q4_0_step_plan(qd.make_q4_0_ops([(w, x, y, 64, 128, 0)]), 1, ws, ws.numel())
    assert e.value.status == qd.QD_ESHAPE
    with pytest.raises(qd.QDError) as e:   # f32 output must be 4-byte aligned
        qd.qgemv_q4_0_step_plan(qd.make_q4_0_ops([(w, x, y + 2, 64, 256, 0)]), 1, ws, ws.numel())
    assert e.value.status == qd.QD_EALIGN
    with pytest.raises(qd.QDError) as e:   # output aliasing the weights
        qd.qgemv_q4_0_step_plan(qd.make_q4_0_ops([(w, x, w + 64, 64, 256, 0)]), 1, ws, ws.numel())
    assert e.value.status == qd.QD_EINVAL
    plan = qd.qgemv_q4_0_step_plan(qd.make_q4_0_ops([(w, x, y, 64, 256, 0)]), 1, ws, ws.numel())
    # a Q4_0 plan is not an affine plan, and the reverse
    assert qd.lib().qgemv_affine_i8_g64_step_run(qd.ctypes.byref(plan), None) == qd.QD_EINVAL
    qd.qgemv_q4_0_step_run(plan)
    assert qd.qgemv_q4_0_step_check(plan) == 0
