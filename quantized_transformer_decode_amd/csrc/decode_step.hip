// decode_step.hip -- one persistent launch for a whole decode step's
// affine-INT8 g64 GEMVs, in stage order (M = 1).
//
// turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step
// encodes every projection GEMV of a generated token, in decoder order, into
// one command pass.  Here the whole sequence is one kernel launch: stage s+1
// (e.g. o after q/k/v, down after gate/up) reads its inputs only after every
// workgroup has finished stage s, so the op order is kept, while the weight
// stream never stops: compute waves load the next stage's weights into
// registers before waiting for the current stage's input.
//
// Exchange between stages.  Inputs travel as tagged 32-bit words
// (stage tag << 16 | BF16 bits) written through to the device coherence
// point with agent-scope stores and polled with agent-scope loads, so one
// store/load round trip carries both the data and the "ready" signal.  A
// workgroup publishes its slice of stage s+1's inputs only after all of its
// compute waves are done with stage s; a consumer therefore sees a complete
// input only once every workgroup has finished stage s.  Tags are
// (epoch + stage) mod 2^16 with the epoch advanced by the stage count per
// launch, so a word left from the previous launch never matches.
//
// Workgroup layout: wave 0 is the poller (publishes, polls the next input
// into LDS as fp32, hands it to the compute waves through an LDS flag);
// waves 1..NCW compute.  The grid is exactly one workgroup per CU and every
// workgroup must be resident (the plan records the grid size; a launch with
// another grid size returns without work and sets the error word).  Every
// wait is bounded; on time-out the error word is set and the kernel runs to
// completion with whatever data it has.
#include "qd_device.h"
#include "qd_internal.h"
#include "qd_step.h"

namespace qd {
namespace {


constexpr int NCW = 8;             // compute waves per workgroup
constexpr int kThreads = (NCW + 1) * kWave;
// Items (1 KiB row chunks) per register group; two groups are in flight per
// wave.  Three covers a wave's share of a layer stage of 0.6B-1.7B decoders
// (1-3 items); larger groups mostly re-read past-the-end items, which delays
// the stage hand-off more than the deeper stream helps the LM-head stage.
constexpr int G = 3;
constexpr unsigned kPollLimit = 1u << 18;   // global polls (~1 us each)
constexpr unsigned kLdsSpinLimit = 1u << 27;

__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
  return __hip_atomic_load((const QD_GLOBAL uint32_t *)p, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent64(const uint64_t *p) {
  return __hip_atomic_load((const QD_GLOBAL uint64_t *)p, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v) {
  __hip_atomic_store((QD_GLOBAL uint32_t *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS flag access between the waves of one workgroup.  Relaxed on purpose:
// LDS executes one wave's operations in issue order, and a release/acquire
// here would also wait for the wave's outstanding global loads (the weight
// prefetch).  The signal fences only stop the compiler from moving LDS data
// accesses across the flag access.
__device__ __forceinline__ int lds_ld(const int *p) {
  const int v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return v;
}

// LDS layout of a staged input: each op's input occupies chunks*1024 floats
// (whole chunks) in the xswz layout.
constexpr int kPubRing = 32;  // stages of publish values kept in LDS ahead of use

struct Shared {
  int xready;        // stages whose input is staged in LDS
  int done;          // compute-wave stage completions
  uint32_t epoch;
  uint32_t pub[kPubRing][64];  // this workgroup's slice of stage s's input at [s % kPubRing]
};

// The rows one compute wave owns in stage s: [lo, hi) of the stage's
// concatenated row space.
__device__ __forceinline__ void wave_rows(const StepStage &st, int gw, int nw, int &lo, int &hi) {
  lo = (int)(((int64_t)st.rows_total * gw) / nw);
  hi = (int)(((int64_t)st.rows_total * (gw + 1)) / nw);
}

struct OpView {
  const QD_GLOBAL uint8_t *w;
  QD_GLOBAL uint16_t *y;
  int rows, cols, row_base, row_end;
};

// Walks the items of one group: row (in the stage's row space) and chunk of
// each item, advancing incrementally (one division per group) and loading an
// op's descriptor only when the walk crosses into the next op.  Everything
// here is wave-uniform and lives in scalar registers.
struct Walk {
  int n, row, ch, chunks, o;
  int op0, scols;  // the stage's first op and input width
  OpView op;
};

struct Group {
  uint4 q[G];
  uint16_t sc[G], bi[G];  // raw BF16 bits; combined only when consumed
  Walk start;             // where the group begins (kept from the issue)
  int i0, s;              // the group's first item and its stage
};

// Where a wave is in its stream of items: stage s, item i of that stage.
struct Cursor {
  int s, i;
};


__device__ __forceinline__ int stage_items(const StepStage *stages, int s, int gw, int nw) {
  s = uni(s);
  int lo, hi;
  wave_rows(stages[s], gw, nw, lo, hi);
  return uni((hi - lo) * stages[s].chunks);
}

// first cursor at or after (s, i) that has an item; s == n_stages at the end
__device__ __forceinline__ Cursor normalize(const StepStage *stages, int n_stages, Cursor c,
                                            int gw, int nw) {
  c.s = uni(c.s);
  c.i = uni(c.i);
  while (c.s < n_stages && c.i >= stage_items(stages, c.s, gw, nw)) {
    c.s = uni(c.s + 1);
    c.i = 0;
  }
  return c;
}

__device__ __forceinline__ int op_of_row(const StepOp *ops, const StepStage &st, int row) {
  int o = st.op0;
  for (int k = 1; k < st.nops; ++k)
    if (row >= ops[st.op0 + k].row_base) o = st.op0 + k;
  return uni(o);
}

__device__ __forceinline__ OpView op_view(const StepOp *ops, int o) {
  const StepOp &op = ops[o];
  OpView v;
  v.w = gp(op.w);
  v.y = gp(op.y);
  v.rows = op.rows;
  v.cols = op.cols;
  v.row_base = op.row_base;
  v.row_end = op.row_base + op.rows;
  return v;
}

__device__ __forceinline__ Walk walk_start(const StepOp *ops, const StepStage &st, Cursor c,
                                           int gw, int nw) {
  Walk w;
  int lo, hi;
  wave_rows(st, gw, nw, lo, hi);
  w.chunks = st.chunks;
  w.op0 = st.op0;
  w.scols = st.cols;
  w.n = uni((hi - lo) * w.chunks);
  const int r = uni(c.i / w.chunks);
  w.row = uni(lo + r);
  w.ch = uni(c.i - r * w.chunks);
  w.o = op_of_row(ops, st, w.row);
  w.op = op_view(ops, w.o);
  return w;
}

__device__ __forceinline__ void walk_next(Walk &w, const StepOp *ops) {
  if (++w.ch == w.chunks) {
    w.ch = 0;
    ++w.row;
    if (w.row >= w.op.row_end) w.op = op_view(ops, ++w.o);
  }
}

// Loads for one group.  Every lane issues exactly the same number of loads
// whatever the group holds (items past the end re-read the last item, lanes
// past a row's end re-read its first chunk): the compiler can then wait for
// exactly this group's loads before it is consumed, instead of for every
// load in flight (which would include the next group's prefetch).
__device__ __forceinline__ void issue(Group &g, const StepOp *ops, const StepStage *stages,
                                      Cursor c, int gw, int nw, int lane) {
  c.s = uni(c.s);
  c.i = uni(c.i);
  Walk wk = walk_start(ops, stages[c.s], c, gw, nw);
  g.start = wk;
  g.i0 = c.i;
  g.s = c.s;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const int lrow = wk.row - wk.op.row_base;
    int col = wk.ch * 1024 + lane * 16;
    if (col >= wk.op.cols) col = 0;
    const u32x4 v = __builtin_nontemporal_load(
        (const QD_GLOBAL u32x4 *)(wk.op.w + (size_t)lrow * wk.op.cols + col));
    g.q[k] = make_uint4(v.x, v.y, v.z, v.w);
    const int groups = wk.op.cols >> 6;
    const QD_GLOBAL uint16_t *sc =
        (const QD_GLOBAL uint16_t *)(wk.op.w + (size_t)wk.op.rows * wk.op.cols);
    const size_t gi = (size_t)lrow * groups + (col >> 6);
    g.sc[k] = sc[gi];
    g.bi[k] = sc[(size_t)wk.op.rows * groups + gi];
    if (c.i + k + 1 < wk.n) walk_next(wk, ops);
  }
}

// Compute one group (the items issue() loaded).  rowsum carries a row's
// partial sum across groups.  The walk state comes from the issue, so the
// only memory this touches is LDS and the weights already in registers.
__device__ __forceinline__ void compute(const Group &g, const StepOp *ops, int lane,
                                        const float *xl, float &rowsum) {
  Walk wk = g.start;
  int xkey = -1;
  float4 x0, x1, x2, x3;
  float xs = 0.f;
#pragma unroll
  for (int k = 0; k < G; ++k) {
    if (g.i0 + k < wk.n) {
      const bool valid = wk.ch * 1024 + lane * 16 < wk.op.cols;
      // x depends only on (op, chunk): reload it only when that changes
      const int key = wk.o * 64 + wk.ch;
      if (key != xkey) {
        xkey = key;
        const float *xp = xl + (wk.o - wk.op0) * (wk.chunks * 1024) + wk.ch * 1024 + lane * 4;
        x0 = *(const float4 *)(xp);
        x1 = *(const float4 *)(xp + 256);
        x2 = *(const float4 *)(xp + 512);
        x3 = *(const float4 *)(xp + 768);
        xs = ((x0.x + x0.y) + (x0.z + x0.w)) + ((x1.x + x1.y) + (x1.z + x1.w)) +
             ((x2.x + x2.y) + (x2.z + x2.w)) + ((x3.x + x3.y) + (x3.z + x3.w));
      }
      const float s = bf16_to_f32(g.sc[k]);
      const float b = bf16_to_f32(g.bi[k]);
      float p = fmaf(s, dot16(g.q[k], x0, x1, x2, x3), b * xs);
      if (!valid) p = 0.f;
      rowsum += wave_sum_dpp(p);
      if (wk.ch == wk.chunks - 1) {
        if (lane == 0) wk.op.y[wk.row - wk.op.row_base] = f32_to_bf16(rowsum);
        rowsum = 0.f;
      }
      walk_next(wk, ops);
    }
  }
}

__device__ __forceinline__ void signal_done_through(Shared *sh, int &signalled, int upto) {
  // mark stages [signalled, upto) done for this wave
  if (signalled < upto) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(&sh->done, upto - signalled,
                                                        __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_WORKGROUP);
    signalled = upto;
  }
}

__device__ void compute_wave(const StepOp *__restrict__ ops, const StepStage *__restrict__ stages,
                             int n_stages, Shared *sh, const float *xbuf, int xmax,
                             uint32_t *err) {
  const int lane = threadIdx.x & 63;
  // wave-uniform values kept in scalar registers, so every table lookup of
  // the schedule is a scalar load (it never waits on the vector-load counter
  // that tracks the weight prefetch)
  const int cw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) - 1;
  const int nw = gridDim.x * NCW;
  const int gw = blockIdx.x * NCW + cw;
  int signalled = 0;
  float rowsum = 0.f;
  int have = 0;  // stages known staged
  Group A, B;

  auto enter = [&](int s) {
    signal_done_through(sh, signalled, s);
    unsigned spins = 0;
    while (have <= s) {
      have = lds_ld(&sh->xready);
      if (have > s) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kLdsSpinLimit) {
        if (lane == 0) atomicOr(err, 4u);
        have = s + 1;
      }
    }
  };

  // Two register groups in flight: while one is consumed the next is loading.
  // The prefetch is issued unconditionally (at the end of the stream it
  // re-reads the current group) so the wait before each consume is exact.
  Cursor c = normalize(stages, n_stages, Cursor{0, 0}, gw, nw);
  if (c.s < n_stages) {
    issue(A, ops, stages, c, gw, nw, lane);
    while (true) {
      const Cursor n1 = normalize(stages, n_stages, Cursor{c.s, c.i + G}, gw, nw);
      issue(B, ops, stages, n1.s < n_stages ? n1 : c, gw, nw, lane);
      enter(c.s);
      compute(A, ops, lane, xbuf + (c.s & 1) * xmax, rowsum);
      if (n1.s >= n_stages) break;
      signal_done_through(sh, signalled, n1.s);  // as soon as a stage is finished
      c = n1;
      const Cursor n2 = normalize(stages, n_stages, Cursor{c.s, c.i + G}, gw, nw);
      issue(A, ops, stages, n2.s < n_stages ? n2 : c, gw, nw, lane);
      enter(c.s);
      compute(B, ops, lane, xbuf + (c.s & 1) * xmax, rowsum);
      if (n2.s >= n_stages) break;
      signal_done_through(sh, signalled, n2.s);
      c = n2;
    }
  }
  signal_done_through(sh, signalled, n_stages);
}

// This workgroup's slice of a stage's inputs (all ops back to back, m*cols
// words each): words [a, b) with a = j * 2^lg, at most 64 words, one per
// lane.  Loaded ahead of time so the publish itself is a single store.
struct PubSlice {
  int a, b;
  uint32_t v;  // word a + lane
};

__device__ __forceinline__ uint32_t input_word(const StepOp *ops, const StepStage &st, int m,
                                               int i) {
  const int w = m * st.cols;
  const int k = i / w;
  return (uint32_t)gp(ops[st.op0 + k].x)[i - k * w];
}

__device__ __forceinline__ PubSlice pub_load(const StepOp *ops, const StepStage &st, int m,
                                             int lane) {
  PubSlice p;
  const int words = st.words;
  p.a = (int)blockIdx.x << st.lg;
  p.b = min(p.a + (1 << st.lg), words);
  p.v = (p.a + lane < p.b) ? input_word(ops, st, m, p.a + lane) : 0u;
  return p;
}

// Everything the poller needs to poll one stage's input and to publish its
// own slice of it, resolved from the tables one stage ahead (scalar loads
// are never on the critical path).
constexpr int kReplicas = 8;  // copies of each published slice (one per XCD)

struct StagePlan {
  const uint64_t *src;  // this workgroup's replica of the staging, 64-bit words
  uint32_t *stg;        // staging, as words (publishing)
  int f0, f1;           // 64-bit words this workgroup polls: [f0, f1)
  int k0, k1;           // ops (within the stage) those words belong to
  int wpo;              // words per op
  int xstride;          // LDS floats per op (whole 1024-column chunks)
  int pa, pb;           // this workgroup's published words [pa, pb)
  int rstride;          // words between replicas
};

__device__ __forceinline__ StagePlan stage_plan(const StepOp *ops, const StepStage &st, int m) {
  StagePlan p;
  // replicas are spaced by one 64-word line per slice; within a replica the
  // words are dense (word i at offset i)
  const int nsl = ((int)st.words + (1 << st.lg) - 1) >> st.lg;
  p.rstride = nsl * 64;
  // workgroups are dispatched round-robin over the XCDs: blockIdx % 8 reads
  // the replica that only the workgroups of its own XCD read
  p.src = (const uint64_t *)(st.stg + (blockIdx.x % kReplicas) * p.rstride);
  p.stg = st.stg;
  p.wpo = m * st.cols;
  p.xstride = st.chunks * 1024;
  int lo, hi, lo2, hi2;
  wave_rows(st, blockIdx.x * NCW, gridDim.x * NCW, lo, hi);
  wave_rows(st, blockIdx.x * NCW + NCW - 1, gridDim.x * NCW, lo2, hi2);
  if (hi2 <= lo) {  // no rows for this workgroup in this stage
    p.k0 = p.k1 = 0;
    p.f0 = p.f1 = 0;
  } else {
    p.k0 = op_of_row(ops, st, lo) - st.op0;
    p.k1 = op_of_row(ops, st, hi2 - 1) - st.op0;
    p.f0 = (p.k0 * p.wpo) >> 1;
    p.f1 = ((p.k1 + 1) * p.wpo) >> 1;
  }
  p.pa = (int)blockIdx.x << st.lg;
  p.pb = min(p.pa + (1 << st.lg), (int)st.words);
  return p;
}

// Poll the part of a stage's input that this workgroup needs (the inputs of
// the ops its compute waves touch) into LDS as fp32; returns false on
// time-out.  Up to B 64-bit words per lane are in flight per batch.
__device__ bool poll_stage(const StagePlan &pp, uint32_t tag, float *dst, int lane,
                           bool aborted) {
  constexpr int B = 24;
  bool ok = true;
  for (int base = pp.f0; base < pp.f1; base += 64 * B) {
    uint64_t v[B];
    unsigned polls = 0;
    while (true) {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        // only words in range are loaded: clamping the rest to one address
        // would pile every lane's extra loads onto a single cache line
        const int f = base + b * 64 + lane;
        v[b] = f < pp.f1
                   ? ld_agent64(pp.src + f)
                   : ((uint64_t)tag << 48) | ((uint64_t)tag << 16);
      }
      bool ready = true;
#pragma unroll
      for (int b = 0; b < B; ++b)
        ready &= ((uint32_t)(v[b] >> 16) & 0xffffu) == tag &&
                 ((uint32_t)(v[b] >> 48) & 0xffffu) == tag;
      if (__all(ready) || aborted) break;
      if (++polls > kPollLimit) { ok = false; break; }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int f = base + b * 64 + lane;
      if (f < pp.f1) {
        // words 2f, 2f+1 belong to one op (each op's input has an even
        // length) and to the same swizzled float pair
        const int e = 2 * f;
        int k = pp.k0;  // the op holding word e (no division: ops are few)
        while (k < pp.k1 && e >= (k + 1) * pp.wpo) ++k;
        const int r = e - k * pp.wpo;
        *(float2 *)(dst + k * pp.xstride + xswz(r)) =
            make_float2(bf16_to_f32((uint32_t)v[b] & 0xffffu),
                        bf16_to_f32((uint32_t)(v[b] >> 32) & 0xffffu));
      }
    }
    if (!ok) return false;
  }
  return true;
}

__device__ void poller_wave(const StepOp *__restrict__ ops, const StepStage *__restrict__ stages,
                            int n_stages, int m, Shared *sh, float *xbuf, int xmax,
                            uint32_t *err) {
  const int lane = threadIdx.x & 63;
  const uint32_t epoch = sh->epoch;
  // after a first time-out this workgroup stops waiting, so a broken run
  // still ends quickly (with the error word set)
  bool aborted = false;
  // The values this workgroup publishes come from the resident inputs; they
  // are loaded kPubRing stages ahead into an LDS ring so that publishing is
  // an LDS read and a store, never a wait on memory.
  for (int t = 0; t < kPubRing && t < n_stages; ++t) {
    const PubSlice p = pub_load(ops, stages[t], m, lane);
    sh->pub[t][lane] = p.v;
  }
  {
    const PubSlice p0 = pub_load(ops, stages[0], m, lane);
    const StagePlan q0 = stage_plan(ops, stages[0], m);
    if (p0.a + lane < p0.b) {
      const uint32_t w = ((epoch & 0xffffu) << 16) | p0.v;
#pragma unroll
      for (int r = 0; r < kReplicas; ++r)
        st_agent(q0.stg + r * q0.rstride + q0.pa + lane, w);
    }
  }
  PubSlice pending;
  int pending_stage = -1;
  StagePlan cur = stage_plan(ops, stages[0], m);
  StagePlan nxt = cur;
  for (int s = 0; s < n_stages; ++s) {
    const uint32_t tag = (epoch + (uint32_t)s) & 0xffffu;
    // park the value loaded one stage ago (long since arrived)
    if (pending_stage >= 0) sh->pub[pending_stage % kPubRing][lane] = pending.v;
    if (!poll_stage(cur, tag, xbuf + (s & 1) * xmax, lane, aborted)) {
      if (lane == 0) atomicOr(err, 1u);
      aborted = true;
    }
    // hand the staged input to the compute waves (LDS executes this wave's
    // data writes before the flag write)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_store(&sh->xready, s + 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
    // resolve the next stage while the compute waves work
    if (s + 1 < n_stages) nxt = stage_plan(ops, stages[s + 1], m);
    // load stage s + kPubRing's values; they are parked next iteration in the
    // slot of stage s, which was published at the end of the last iteration
    pending_stage = -1;
    if (s + kPubRing < n_stages) {
      pending = pub_load(ops, stages[s + kPubRing], m, lane);
      pending_stage = s + kPubRing;
    }
    // wait for every compute wave to finish stage s, then publish s+1
    unsigned spins = 0;
    while (lds_ld(&sh->done) < (s + 1) * NCW) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kLdsSpinLimit) {
        if (lane == 0) atomicOr(err, 2u);
        break;
      }
    }
    if (s + 1 < n_stages) {
      const uint32_t t1 = ((epoch + (uint32_t)s + 1) & 0xffffu) << 16;
      if (nxt.pa + lane < nxt.pb) {
        const uint32_t w = t1 | sh->pub[(s + 1) % kPubRing][lane];
#pragma unroll
        for (int r = 0; r < kReplicas; ++r)
          st_agent(nxt.stg + r * nxt.rstride + nxt.pa + lane, w);
      }
    }
    cur = nxt;
  }
}

__global__ __launch_bounds__(kThreads) void affine_step_kernel(
    const StepOp *__restrict__ ops, const StepStage *__restrict__ stages, int n_stages,
    int m, int xmax, int nwg, uint32_t *__restrict__ epoch_word, uint32_t *__restrict__ err) {
  if ((int)gridDim.x != nwg) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err, 8u);
    return;
  }
  __shared__ Shared sh;
  extern __shared__ __attribute__((aligned(16))) float xbuf[];  // [2][xmax]
  if (threadIdx.x == 0) {
    sh.xready = 0;
    sh.done = 0;
    sh.epoch = ld_agent(epoch_word);
  }
  __syncthreads();
  if (threadIdx.x < kWave)
    poller_wave(ops, stages, n_stages, m, &sh, xbuf, xmax, err);
  else
    compute_wave(ops, stages, n_stages, &sh, xbuf, xmax, err);
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0) st_agent(epoch_word, sh.epoch + (uint32_t)n_stages);
}

}  // namespace

int step_threads() { return kThreads; }

hipError_t launch_affine_step(const StepOp *ops, const StepStage *stages, int n_stages, int m,
                              int xmax, int nwg, uint32_t *epoch_word, uint32_t *err,
                              size_t lds_bytes, hipStream_t stream) {
  if (lds_bytes > 65536) {
    hipError_t e = hipFuncSetAttribute((const void *)affine_step_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds_bytes);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(affine_step_kernel, dim3(nwg), dim3(kThreads), lds_bytes, stream, ops,
                     stages, n_stages, m, xmax, nwg, epoch_word, err);
  return hipGetLastError();
}

}  // namespace qd
