"""GPU parity of the single-launch decode step (qgemv_affine_i8_g64_step_*)
against the oracle, GEMV by GEMV.

turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step
(the GEMV sequence of one token, in decoder order).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_transformer_decode_amd as qd
import synth
from helpers import DEV, check_bf16_output, dev_bf16, host_bf16_f64, pack_on_device

pytestmark = pytest.mark.gpu


class Step:
    def __init__(self, shapes, key, m=1, share_weights=None):
        """shapes: list of (rows, cols, stage); m token rows.  share_weights:
        optional per-op index of an earlier op whose weights it reuses."""
        self.shapes = shapes
        self.m = m
        self.blobs, self.xbits, self.xs, self.ys = [], [], [], []
        for i, (rows, cols, stage) in enumerate(shapes):
            j = share_weights[i] if share_weights is not None else i
            if j == i:
                tr = synth.affine_triplet(rows, cols, key=(key, i, 0))
                self.blobs.append(pack_on_device(tr))
            else:
                self.blobs.append(self.blobs[j])
            xb = synth.x_bf16(m, cols, key=(key, i, 1))
            self.xbits.append(xb)
            self.xs.append(dev_bf16(xb))
            self.ys.append(torch.full((m, rows), float("nan"), dtype=torch.bfloat16, device=DEV))
        self.ops = qd.make_ops((b, x, y, r, c, s) for (r, c, s), b, x, y in
                               zip(shapes, self.blobs, self.xs, self.ys))
        nbytes = qd.qgemv_affine_i8_g64_step_workspace_bytes(self.ops, m)
        assert nbytes > 0
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        self.plan = qd.qgemv_affine_i8_g64_step_plan(self.ops, m, self.ws, nbytes)
        assert self.plan.m == m

    def run(self):
        qd.qgemv_affine_i8_g64_step_run(self.plan)
        assert qd.qgemv_affine_i8_g64_step_check(self.plan) == 0

    def check(self, sample_rows=None, what=""):
        for i, (rows, cols, stage) in enumerate(self.shapes):
            sel = None
            if sample_rows and rows > sample_rows:
                sel = np.unique(np.concatenate([
                    np.random.default_rng(i).integers(0, rows, sample_rows), [0, rows - 1]]))
            ref = oracle.affine_gemv(self.blobs[i].cpu().numpy(), rows, cols, self.xbits[i],
                                     row_sel=sel)
            assert ref.shape[0] == self.m
            got = host_bf16_f64(self.ys[i])
            if sel is not None:
                got = got[:, sel]
            check_bf16_output(got, ref, f"{what} op {i} ({rows}x{cols}, stage {stage})")


SMALL = [(130, 256, 0), (64, 256, 0), (17, 256, 0),      # three GEMVs sharing a stage
         (256, 130 * 0 + 192, 1),                          # one GEMV, odd width
         (3000, 256, 2), (3000, 256, 2),                   # more rows than waves
         (256, 3072, 3),                                   # several 1 KiB chunks per row
         (1, 64, 4),                                       # a single output
         (5000, 1088, 5)]                                  # partial last chunk


def test_step_small_parity_and_relaunch():
    print("step small", flush=True)
    st = Step(SMALL, key=20)
    st.run()
    st.check(what="first launch")
    # a second launch with new inputs must read the new inputs (tags of the
    # previous launch never match)
    for i, (rows, cols, stage) in enumerate(SMALL):
        xb = synth.x_bf16(1, cols, key=(21, i, 1))
        st.xbits[i] = xb
        st.xs[i].copy_(dev_bf16(xb))
        st.ys[i].fill_(float("nan"))
    torch.cuda.synchronize()
    st.run()
    st.check(what="second launch")


def test_step_graph_replays():
    print("step graph", flush=True)
    st = Step(SMALL[:5], key=22)
    st.run()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            qd.qgemv_affine_i8_g64_step_run(st.plan)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in st.ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert qd.qgemv_affine_i8_g64_step_check(st.plan) == 0
        st.check(what=f"replay {rep}")


# a last stage of one GEMV of >= 2^27 weights runs as a second, streaming
# launch (plan.tail); one exactly at the threshold and one below it
TAIL = [(130, 256, 0), (64, 256, 0), (256, 1024, 1), (131072, 1024, 2)]
NO_TAIL = [(130, 256, 0), (256, 1024, 1), (131071, 1024, 2)]


def test_step_streamed_last_stage_eager_and_graph():
    print("step tail", flush=True)
    st = Step(TAIL, key=24)
    assert st.plan.tail == 1 and st.plan.tail_rows == 131072 and st.plan.tail_cols == 1024
    st.run()
    st.check(sample_rows=64, what="tail eager")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            qd.qgemv_affine_i8_g64_step_run(st.plan)
    torch.cuda.synchronize()
    for rep in range(2):
        for y in st.ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert qd.qgemv_affine_i8_g64_step_check(st.plan) == 0
        st.check(sample_rows=64, what=f"tail replay {rep}")
    nt = Step(NO_TAIL, key=25)
    assert nt.plan.tail == 0
    nt.run()
    nt.check(sample_rows=64, what="below the tail threshold")


def test_step_qwen3_0_6b_full_size_sampled():
    # the full 197-GEMV step of the Qwen3-0.6B-shaped decoder; every GEMV is
    # checked on sampled rows
    print("step qwen3-0.6b", flush=True)
    shapes = [(rows, cols, stage) for (_, _, rows, cols, stage)
              in synth.decode_step_matrices(synth.QWEN3_0_6B)]
    st = Step(shapes, key=23)
    assert st.plan.tail == 1  # the 151936 x 1024 LM head streams on its own
    assert st.plan.group == 3  # 1.25 weight chunks per compute wave and stage
    for _ in range(3):
        st.run()
    st.check(sample_rows=48, what="qwen3-0.6b")


def test_step_group_of_four_parity_and_relaunch():
    # stages that give each compute wave more than three weight chunks on
    # average take register groups of four: gate/up 2 x 6144 x 2048, down
    # 2048 x 6144, then a 2048 x 2048 GEMV, every output row checked
    print("step groups of four", flush=True)
    shapes = [(6144, 2048, 0), (6144, 2048, 0), (2048, 6144, 1), (2048, 2048, 2)]
    st = Step(shapes, key=29)
    assert st.plan.group == 4 and st.plan.tail == 0
    for _ in range(3):
        st.run()
    st.check(what="groups of four")


def test_step_qwen3_1_7b_full_size_sampled():
    # the full Qwen3-1.7B-shaped step at one token row (groups of four; one
    # layer's matrices shared by all 28 layers), every GEMV checked on
    # sampled rows
    print("step qwen3-1.7b m=1", flush=True)
    mats = synth.decode_step_matrices(synth.QWEN3_1_7B)
    shapes = [(rows, cols, stage) for (_, _, rows, cols, stage) in mats]
    first = {}
    share = []
    for i, (layer, name, rows, cols, stage) in enumerate(mats):
        first.setdefault(name, i)
        share.append(first[name])
    st = Step(shapes, key=41, m=1, share_weights=share)
    assert st.plan.tail == 1 and st.plan.group == 4
    for _ in range(2):
        st.run()
    st.check(sample_rows=24, what="qwen3-1.7b m=1")


def test_step_plan_rejects_bad_ops():
    t = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    base = t.data_ptr()
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=DEV)
    ok = [(base, base + 65536, base + 131072, 64, 128, 0)]
    with pytest.raises(qd.QDError) as e:   # first stage must be 0
        qd.qgemv_affine_i8_g64_step_plan(qd.make_ops([(base, base + 65536, base + 131072, 64, 128, 1)]),
                                         1, ws, ws.numel())
    assert e.value.status == qd.QD_EINVAL
    with pytest.raises(qd.QDError) as e:   # ops of one stage must share cols
        qd.qgemv_affine_i8_g64_step_plan(qd.make_ops(ok + [(base, base + 65536, base + 200000, 64, 192, 0)]),
                                         1, ws, ws.numel())
    assert e.value.status == qd.QD_ESHAPE
    with pytest.raises(qd.QDError) as e:   # output aliasing an input
        qd.qgemv_affine_i8_g64_step_plan(qd.make_ops(ok + [(base, base + 131072, base + 300000, 64, 64, 1)]),
                                         1, ws, ws.numel())
    assert e.value.status == qd.QD_EINVAL
    for m in (0, 5):                        # 1..4 token rows
        with pytest.raises(qd.QDError) as e:
            qd.qgemv_affine_i8_g64_step_plan(qd.make_ops(ok), m, ws, ws.numel())
        assert e.value.status == qd.QD_EINVAL
    with pytest.raises(qd.QDError) as e:   # workspace too small
        qd.qgemv_affine_i8_g64_step_plan(qd.make_ops(ok), 1, ws, 512)
    assert e.value.status == qd.QD_EINVAL


# Several token rows (one persistent kernel per row count): every op's x is
# [m, cols] and y [m, rows]; the staged input holds only the ops a
# workgroup has rows in.
@pytest.mark.parametrize("m", [2, 3, 4])
def test_step_rows_small_parity_and_relaunch(m):
    print(f"step m={m} small", flush=True)
    st = Step(SMALL, key=30 + m, m=m)
    st.run()
    st.check(what=f"m={m} first launch")
    for i, (rows, cols, stage) in enumerate(SMALL):
        xb = synth.x_bf16(m, cols, key=(35 + m, i, 1))
        st.xbits[i] = xb
        st.xs[i].copy_(dev_bf16(xb))
        st.ys[i].fill_(float("nan"))
    torch.cuda.synchronize()
    st.run()
    st.check(what=f"m={m} second launch")


def test_step_rows_graph_and_streamed_tail():
    # m = 4 with a last stage streamed on its own (the matrix-core GEMV at
    # four rows), eager and as graph replays
    print("step m=4 tail", flush=True)
    st = Step(TAIL, key=39, m=4)
    assert st.plan.tail == 1
    st.run()
    st.check(sample_rows=64, what="m=4 tail eager")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            qd.qgemv_affine_i8_g64_step_run(st.plan)
    torch.cuda.synchronize()
    for rep in range(2):
        for y in st.ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert qd.qgemv_affine_i8_g64_step_check(st.plan) == 0
        st.check(sample_rows=64, what=f"m=4 tail replay {rep}")


def test_step_rows_qwen3_1_7b_full_size_sampled():
    # the full Qwen3-1.7B-shaped step at four token rows (one layer's
    # matrices shared by all 28 layers), every GEMV checked on sampled rows
    print("step qwen3-1.7b m=4", flush=True)
    mats = synth.decode_step_matrices(synth.QWEN3_1_7B)
    shapes = [(rows, cols, stage) for (_, _, rows, cols, stage) in mats]
    first = {}
    share = []
    for i, (layer, name, rows, cols, stage) in enumerate(mats):
        first.setdefault(name, i)
        share.append(first[name])
    st = Step(shapes, key=40, m=4, share_weights=share)
    assert st.plan.tail == 1
    for _ in range(2):
        st.run()
    st.check(sample_rows=24, what="qwen3-1.7b m=4")
