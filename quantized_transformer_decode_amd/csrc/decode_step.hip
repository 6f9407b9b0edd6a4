// decode_step.hip -- one persistent launch for a whole decode step's
// GEMVs, in stage order: affine-INT8 g64 ops (BF16, 1..4 token rows), or
// Q4_0 ops (f32, one row: the Whisper decoder's projections).
//
// turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step
// encodes every projection GEMV of a generated token, in decoder order, into
// one command pass.  Here the whole sequence is one kernel launch: stage s+1
// (e.g. o after q/k/v, down after gate/up) reads its inputs only after every
// workgroup has finished stage s, so the op order is kept, while the weight
// stream never stops: compute waves load the next stage's weights into
// registers before waiting for the current stage's input.
//
// Exchange between stages.  After all of its compute waves are done with
// stage s, a workgroup stores its slice of stage s+1's input (dense words,
// two BF16 each) with agent-scope stores, waits for their acknowledgement,
// and arrives at the stage's barrier: one agent-scope atomic on the counter
// of its group (workgroup b -> group b % 8, one group per XCD); the group's
// last arrival increments the stage's global counter, and the last of those
// writes the stage's tag into every workgroup's own 128-byte release line.
// Each workgroup polls only its own line, then reads the inputs it needs
// with agent-scope loads (all in flight at once).  No line is polled by
// more than one workgroup and no counter takes more than 32 atomics per
// stage: a single shared counter or flag array, polled by every workgroup,
// measured about twice as slow per stage on this part.  Tags are epoch +
// stage with the epoch advanced by the stage count per launch; counters
// only grow (each launch adds the same amounts, so arrivals are counted
// modulo the group sizes), so nothing is cleared between launches or graph
// replays.  The first stage's input is read straight from the ops' inputs,
// which are written before the launch.
//
// Q4_0 ops: a work item is 64 blocks (2048 columns) of one row, lane l
// holding block l in the 20-byte window that starts 2 bytes early for odd
// blocks (the Q4_0 GEMV's load form; a row's block count is a multiple of 8,
// so a block's parity is its lane's); the staged input goes to LDS as fp32
// in a layout where lane l's eight float4 of block l are conflict-free; the
// exchange words are the f32 inputs themselves.
//
// Workgroup layout: wave 0 is the poller (publishes, polls the next input
// into LDS as fp32, hands it to the compute waves through an LDS flag);
// waves 1..kNcw compute.  The grid is exactly one workgroup per CU and every
// workgroup must be resident (the plan records the grid size; a launch with
// another grid size returns without work and sets the error word).  Every
// wait is bounded; on time-out the error word is set and the kernel runs to
// completion with whatever data it has.
#include "qd_device.h"
#include "qd_internal.h"
#include "qd_step.h"

namespace qd {
namespace {


// Compute waves per workgroup: twelve for affine ops at one token row
// (against eight: the Qwen3-1.7B step 0.868 -> 0.820 ms, the 0.6B step
// unchanged), eight for Q4_0 ops (twelve: the Whisper-large step 0.70 ->
// 0.73 ms) and for several token rows (their x and row sums take registers
// that twelve waves per CU cannot spare).
template <bool Q4, int MT>
constexpr int kNcw = (Q4 || MT > 1) ? 8 : 12;
template <bool Q4, int MT>
constexpr int kThreads = (kNcw<Q4, MT> + 1) * kWave;
// Several token rows stage only the ops a workgroup has rows in (a stage's
// whole input would not fit in LDS); one row stages every op of the stage at
// a fixed place (the single-row kernel is at its register limit).
template <bool Q4, int MT>
constexpr bool kCompact = MT > 1;
// Items (1 KiB row chunks) per register group, NG: two groups are in flight
// per wave.  Three covers a wave's share of a layer stage of a 0.6B decoder
// (1-3 items); larger groups there mostly re-read past-the-end items, which
// delays the stage hand-off more than the deeper stream helps.  A plan whose
// stages give the waves more (a 1.7B decoder: up to 8 items in its gate/up
// stage) takes four, the most the single-row kernel's 128 VGPRs hold.
constexpr int kGroupItems = 3;
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

// LDS layout of a staged input, op k at (k - kbase) * xstride floats:
// - one token row: kbase = 0 (every op of the stage), whole 1024-column
//   chunks of fp32 in the xswz layout (Q4_0: 2048-column items of fp32 in
//   the xq4 layout);
// - m > 1 token rows: kbase = the first op this workgroup has rows in, the
//   BF16 values as published, in the xswz order, token row t at
//   t * chunks * 1024 elements (fp32 would not fit a 6144-wide input of
//   four rows twice).
constexpr int kPubRing = 2;   // stages of publish values kept in LDS ahead of use

struct Shared {
  int xready;        // stages whose input is staged in LDS
  int done;          // compute-wave stage completions
  int arrived;       // stages whose barrier this workgroup has arrived at
  uint32_t epoch;
  int xk0[2];        // kbase of stage s's staged input, at [s & 1]
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

// Columns of one work item: a 1 KiB row chunk of affine codes, or 64 Q4_0
// blocks.
template <bool Q4>
constexpr int kItemCols = Q4 ? 2048 : 1024;

template <bool Q4, int NG>
struct Loads;
template <int NG>
struct Loads<false, NG> {
  uint4 q[NG];
  uint16_t sc[NG], bi[NG];  // raw BF16 bits; combined only when consumed
};
template <int NG>
struct Loads<true, NG> {
  u32x4 w4[NG];             // the 20-byte block windows
  uint32_t w1[NG];
};

template <bool Q4, int NG>
struct Group : Loads<Q4, NG> {
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
template <bool Q4, int NG>
__device__ __forceinline__ void issue_walk(Group<Q4, NG> &g, const StepOp *ops, Walk wk, Cursor c,
                                           int lane) {
  c.s = uni(c.s);
  c.i = uni(c.i);
  g.start = wk;
  g.i0 = c.i;
  g.s = c.s;
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int lrow = wk.row - wk.op.row_base;
    if constexpr (Q4) {
      // block ch*64 + lane of the row (lanes past the row re-read block 0 or
      // 1, keeping their parity)
      const int nb = wk.op.cols >> 5;
      int blk = wk.ch * 64 + lane;
      if (blk >= nb) blk = lane & 1;
      const QD_GLOBAL uint8_t *p =
          wk.op.w + 18 * ((size_t)lrow * nb + blk) - 2 * (lane & 1);
      g.w4[k] = __builtin_nontemporal_load((const QD_GLOBAL u32x4 *)p);
      g.w1[k] = __builtin_nontemporal_load((const QD_GLOBAL uint32_t *)(p + 16));
    } else {
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
    }
    if (c.i + k + 1 < wk.n) walk_next(wk, ops);
  }
}

template <bool Q4, int NG>
__device__ __forceinline__ void issue(Group<Q4, NG> &g, const StepOp *ops, const StepStage *stages,
                                      Cursor c, int gw, int nw, int lane) {
  c.s = uni(c.s);
  c.i = uni(c.i);
  issue_walk(g, ops, walk_start(ops, stages[c.s], c, gw, nw), c, lane);
}

// Compute one group (the items issue() loaded).  rowsum carries a row's
// partial sum across groups.  The walk state comes from the issue, so the
// only memory this touches is LDS and the weights already in registers.
// Q4_0 staging layout inside one 2048-column item: element 32*blk + 4*j4 + r
// at float4 slot 8*blk + (j4 ^ ((blk >> 1) & 7)).  Lane blk reads its eight
// slots; sixteen consecutive lanes then cover all 64 banks, and so do the
// poller's writes of consecutive elements.
__device__ __forceinline__ int xq4(int e) {
  const int c = e & ~2047, r = e & 2047;
  const int blk = r >> 5, j4 = (r >> 2) & 7;
  return c + ((8 * blk + (j4 ^ ((blk >> 1) & 7))) << 2) + (r & 3);
}

// One Q4_0 work item: lane l holds block ch*64 + l (20-byte window w, odd
// parity = lane & 1) against x[32 l .. 32 l + 31] in registers; returns
// d * (sum_j q_j x_j - 8 * sum_j x_j).
__device__ __forceinline__ float q4_item(const u32x4 w4, uint32_t w1, int lane,
                                         const float4 (&xq)[8], float xs) {
  const uint32_t w[5] = {w4.x, w4.y, w4.z, w4.w, w1};
  const bool odd = lane & 1;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t nib = odd ? w[k + 1] : __builtin_amdgcn_alignbyte(w[k + 1], w[k], 2);
    const uint32_t lo = nib & 0x0f0f0f0fu, hi = (nib >> 4) & 0x0f0f0f0fu;
    // low nibbles: elements 4k..4k+3; high nibbles: 16+4k..16+4k+3
    s0 = fmaf(ubyte<0>(lo), xq[k].x, s0);
    s0 = fmaf(ubyte<1>(lo), xq[k].y, s0);
    s0 = fmaf(ubyte<2>(lo), xq[k].z, s0);
    s0 = fmaf(ubyte<3>(lo), xq[k].w, s0);
    s1 = fmaf(ubyte<0>(hi), xq[4 + k].x, s1);
    s1 = fmaf(ubyte<1>(hi), xq[4 + k].y, s1);
    s1 = fmaf(ubyte<2>(hi), xq[4 + k].z, s1);
    s1 = fmaf(ubyte<3>(hi), xq[4 + k].w, s1);
  }
  const float d = f16_to_f32(odd ? (w[0] >> 16) : (w[0] & 0xffffu));
  return d * fmaf(-8.f, xs, s0 + s1);
}

template <int NG>
__device__ __forceinline__ void compute_q4(const Group<true, NG> &g, const StepOp *ops, int lane,
                                           const float *xl, int k0, float &rowsum) {
  {
    Walk wk = g.start;
    int xkey = -1;
    float4 xq[8];
    float xs = 0.f;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      if (g.i0 + k < wk.n) {
        const bool valid = wk.ch * 64 + lane < (wk.op.cols >> 5);
        const int key = wk.o * 64 + wk.ch;
        if (key != xkey) {
          xkey = key;
          const float *xp = xl + (wk.o - wk.op0 - k0) * (wk.chunks * 2048) + wk.ch * 2048;
          xs = 0.f;
#pragma unroll
          for (int j4 = 0; j4 < 8; ++j4) {
            xq[j4] = *(const float4 *)(xp + ((8 * lane + (j4 ^ ((lane >> 1) & 7))) << 2));
            xs += (xq[j4].x + xq[j4].y) + (xq[j4].z + xq[j4].w);
          }
        }
        float p = q4_item(g.w4[k], g.w1[k], lane, xq, xs);
        if (!valid) p = 0.f;
        rowsum += wave_sum_dpp(p);
        if (wk.ch == wk.chunks - 1) {
          if (lane == 0) ((QD_GLOBAL float *)wk.op.y)[wk.row - wk.op.row_base] = rowsum;
          rowsum = 0.f;
        }
        if (g.i0 + k + 1 < wk.n) walk_next(wk, ops);
      }
    }
  }
}

// 16 codes (one 16-byte load) against MT token rows of 16 activations each:
// the codes converted once.
template <int MT>
__device__ __forceinline__ void dot16_rows(const uint4 q, const float4 (&x)[MT][4],
                                           float (&d)[MT]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int t = 0; t < MT; ++t) d[t] = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float c0 = ubyte<0>(w[k]), c1 = ubyte<1>(w[k]), c2 = ubyte<2>(w[k]),
                c3 = ubyte<3>(w[k]);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      d[t] = fmaf(c0, x[t][k].x, d[t]);
      d[t] = fmaf(c1, x[t][k].y, d[t]);
      d[t] = fmaf(c2, x[t][k].z, d[t]);
      d[t] = fmaf(c3, x[t][k].w, d[t]);
    }
  }
}

template <int MT, int NG>
__device__ __forceinline__ void compute_affine(const Group<false, NG> &g, const StepOp *ops,
                                               int lane, const float *xl, int k0,
                                               float (&rowsum)[MT]) {
  if constexpr (MT == 1) {
    Walk wk = g.start;
    int xkey = -1;
    float4 x0, x1, x2, x3;
    float xs = 0.f;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      if (g.i0 + k < wk.n) {
        const bool valid = wk.ch * 1024 + lane * 16 < wk.op.cols;
        // x depends only on (op, chunk): reload it only when that changes
        const int key = wk.o * 64 + wk.ch;
        if (key != xkey) {
          xkey = key;
          const float *xp =
              xl + (wk.o - wk.op0 - k0) * (wk.chunks * 1024) + wk.ch * 1024 + lane * 4;
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
        rowsum[0] += wave_sum_dpp(p);
        if (wk.ch == wk.chunks - 1) {
          if (lane == 0) wk.op.y[wk.row - wk.op.row_base] = f32_to_bf16(rowsum[0]);
          rowsum[0] = 0.f;
        }
        // past the group's last valid item there is no next descriptor to read
        // (after the plan's last op the table ends)
        if (g.i0 + k + 1 < wk.n) walk_next(wk, ops);
      }
    }
  } else {
    // MT token rows: row t of an op's staged input at t * chunks * 1024
    Walk wk = g.start;
    int xkey = -1;
    float4 x[MT][4];
    float xs[MT];
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      if (g.i0 + k < wk.n) {
        const bool valid = wk.ch * 1024 + lane * 16 < wk.op.cols;
        const int key = wk.o * 64 + wk.ch;
        if (key != xkey) {
          xkey = key;
          const uint16_t *xp = (const uint16_t *)(xl + (wk.o - wk.op0 - k0) *
                                                           (MT * wk.chunks * 512)) +
                               wk.ch * 1024 + lane * 4;
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const uint16_t *xt = xp + t * (wk.chunks * 1024);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const u32x2 w = *(const u32x2 *)(xt + 256 * j);
              x[t][j] = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                                    __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
            }
            xs[t] = ((x[t][0].x + x[t][0].y) + (x[t][0].z + x[t][0].w)) +
                    ((x[t][1].x + x[t][1].y) + (x[t][1].z + x[t][1].w)) +
                    ((x[t][2].x + x[t][2].y) + (x[t][2].z + x[t][2].w)) +
                    ((x[t][3].x + x[t][3].y) + (x[t][3].z + x[t][3].w));
          }
        }
        const float s = bf16_to_f32(g.sc[k]);
        const float b = bf16_to_f32(g.bi[k]);
        float d[MT];
        dot16_rows<MT>(g.q[k], x, d);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          float p = fmaf(s, d[t], b * xs[t]);
          if (!valid) p = 0.f;
          rowsum[t] += wave_sum_dpp(p);
        }
        if (wk.ch == wk.chunks - 1) {
          if (lane < MT) {
            float v = rowsum[0];
#pragma unroll
            for (int t = 1; t < MT; ++t) v = lane == t ? rowsum[t] : v;
            wk.op.y[(size_t)lane * wk.op.rows + (wk.row - wk.op.row_base)] = f32_to_bf16(v);
          }
#pragma unroll
          for (int t = 0; t < MT; ++t) rowsum[t] = 0.f;
        }
        if (g.i0 + k + 1 < wk.n) walk_next(wk, ops);
      }
    }
  }
}

template <bool Q4, int MT, int NG>
__device__ __forceinline__ void compute(const Group<Q4, NG> &g, const StepOp *ops, int lane,
                                        const float *xl, int k0, float (&rowsum)[MT]) {
  if constexpr (Q4)
    compute_q4<NG>(g, ops, lane, xl, k0, rowsum[0]);
  else
    compute_affine<MT, NG>(g, ops, lane, xl, k0, rowsum);
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

// (forced inline, as the poller below: two kernels share it, and a call would
// move the register groups through scratch memory)
template <bool Q4, int MT, int NG>
__device__ __forceinline__ void compute_wave(const StepOp *__restrict__ ops,
                                             const StepStage *__restrict__ stages,
                                             int n_stages, Shared *sh, const float *xbuf,
                                             int xmax, uint32_t *err) {
  const int lane = threadIdx.x & 63;
  // wave-uniform values kept in scalar registers, so every table lookup of
  // the schedule is a scalar load (it never waits on the vector-load counter
  // that tracks the weight prefetch)
  const int cw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) - 1;
  const int nw = gridDim.x * kNcw<Q4, MT>;
  const int gw = blockIdx.x * kNcw<Q4, MT> + cw;
  int signalled = 0;
  float rowsum[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) rowsum[t] = 0.f;
  int have = 0;  // stages known staged
  Group<Q4, NG> A, B;

  auto enter = [&](int s) {
    signal_done_through(sh, signalled, s);
    unsigned spins = 0;
    while (have <= s) {
      have = lds_ld(&sh->xready);
      if (have > s) break;
      if (++spins > kLdsSpinLimit) {
        if (lane == 0) atomicOr(err, 4u);
        have = s + 1;
      }
    }
  };

  // the first op of stage s's staged input (read after the stage is staged)
  auto staged_base = [&](int s) -> int {
    if constexpr (kCompact<Q4, MT>)
      return uni(sh->xk0[s & 1]);
    else
      return 0;
  };

  auto wait_arrived = [&](int t) {
    unsigned spins = 0;
    while (lds_ld(&sh->arrived) < t) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kLdsSpinLimit) {
        if (lane == 0) atomicOr(err, 4u);
        break;
      }
    }
  };

  // Two register groups: while one is consumed the next is loading.  Inside
  // a stage the next group is issued before the current one is consumed.
  // The first group of the next stage is issued only once this workgroup
  // has arrived at that stage's barrier: the burst then drains while the
  // barrier completes, instead of queueing in front of the loads on the
  // hand-off's critical path (the input read, the arrival, the release
  // poll), which this CU issues through the same memory pipeline.  Both
  // paths compute in their own branch, so each waits for exactly the loads
  // it consumes.
  Cursor c = normalize(stages, n_stages, Cursor{0, 0}, gw, nw);
  auto run = [&](Group<Q4, NG> &cur, Group<Q4, NG> &nxt) __attribute__((always_inline)) -> bool {
    const Cursor n1 = normalize(stages, n_stages, Cursor{c.s, c.i + NG}, gw, nw);
    if (n1.s == c.s) {
      issue(nxt, ops, stages, n1, gw, nw, lane);
      enter(c.s);
      compute<Q4, MT, NG>(cur, ops, lane, xbuf + (c.s & 1) * xmax, staged_base(c.s), rowsum);
    } else {
      enter(c.s);
      compute<Q4, MT, NG>(cur, ops, lane, xbuf + (c.s & 1) * xmax, staged_base(c.s), rowsum);
      if (n1.s >= n_stages) return false;
      signal_done_through(sh, signalled, n1.s);  // as soon as a stage is finished
      // the next stage's schedule lookups (dependent scalar loads) while the
      // hand-off completes; only the weight loads wait for the arrival
      const Walk wn = walk_start(ops, stages[uni(n1.s)], n1, gw, nw);
      wait_arrived(c.s + 1);
      issue_walk(nxt, ops, wn, n1, lane);
    }
    c = n1;
    return true;
  };
  if (c.s < n_stages) {
    issue(A, ops, stages, c, gw, nw, lane);
    while (run(A, B) && run(B, A)) {
    }
  }
  signal_done_through(sh, signalled, n_stages);
}

// This workgroup's slice of a stage's input words (all ops back to back,
// m*cols/2 words each, two BF16 per word): words [a, b) with a = j * 2^lg,
// at most 64 words, one per lane.  Loaded ahead of time so that publishing
// is an LDS read and a store.
struct PubSlice {
  int a, b;
  uint32_t v;  // word a + lane
};

template <bool Q4>
__device__ __forceinline__ uint32_t input_word(const StepOp *ops, const StepStage &st, int m,
                                               int i) {
  const int w = Q4 ? m * st.cols : m * st.cols / 2;  // words per op (f32, or BF16 pairs)
  const int k = i / w;
  const QD_GLOBAL uint32_t *x = (const QD_GLOBAL uint32_t *)gp(ops[st.op0 + k].x);
  return x[i - k * w];
}

template <bool Q4>
__device__ __forceinline__ PubSlice pub_load(const StepOp *ops, const StepStage &st, int m,
                                             int lane) {
  PubSlice p;
  const int words = st.words;
  p.a = (int)blockIdx.x << st.lg;
  p.b = min(p.a + (1 << st.lg), words);
  p.v = (p.a + lane < p.b) ? input_word<Q4>(ops, st, m, p.a + lane) : 0u;
  return p;
}

// Everything the poller needs to read one stage's input and to publish its
// own slice of it, resolved from the tables one stage ahead.
struct StagePlan {
  uint32_t *data;       // the stage's input words
  int f0, f1;           // 64-bit words this workgroup reads: [f0, f1)
  int k0, k1;           // ops (within the stage) those words belong to
  int kbase;            // the op staged first in LDS: k0, or 0 (one token row)
  int epo;              // input elements per op
  int xstride;          // LDS floats per op (whole 1024-column chunks)
  int pa, pb;           // this workgroup's published words [pa, pb)
};

template <bool Q4, int MT>
__device__ __forceinline__ StagePlan stage_plan(const StepOp *ops, const StepStage &st, int m) {
  // 64-bit exchange words: four BF16 inputs, or two f32 (Q4_0)
  constexpr int kLgPer64 = Q4 ? 1 : 2;
  StagePlan p;
  p.data = st.data;
  p.epo = m * st.cols;
  p.xstride = MT == 1 ? st.chunks * kItemCols<Q4> : MT * st.chunks * 512;
  int lo, hi, lo2, hi2;
  constexpr int NCW = kNcw<Q4, MT>;
  wave_rows(st, blockIdx.x * NCW, gridDim.x * NCW, lo, hi);
  wave_rows(st, blockIdx.x * NCW + NCW - 1, gridDim.x * NCW, lo2, hi2);
  if (hi2 <= lo) {  // no rows for this workgroup in this stage
    p.k0 = p.k1 = 0;
    p.f0 = p.f1 = 0;
  } else {
    p.k0 = op_of_row(ops, st, lo) - st.op0;
    p.k1 = op_of_row(ops, st, hi2 - 1) - st.op0;
    p.f0 = (p.k0 * p.epo) >> kLgPer64;
    p.f1 = ((p.k1 + 1) * p.epo) >> kLgPer64;
  }
  p.kbase = kCompact<Q4, MT> ? p.k0 : 0;
  p.pa = (int)blockIdx.x << st.lg;
  p.pb = min(p.pa + (1 << st.lg), (int)st.words);
  return p;
}

// One 64-bit input word into LDS as fp32: four BF16 elements (xswz layout),
// or two f32 elements (Q4_0, xq4 layout).
// Element index in LDS (BF16 units, relative to the op) of element r of an
// op's MT-row input: token row t = r / cols at t * tstride, then the
// column's xswz slot (the fp32 layout's order, two bytes per element: lane
// l's 16 columns of a chunk are its four 8-byte pieces at 4 l + 256 j).
template <int MT>
__device__ __forceinline__ int x_pos(int r, int cols, int tstride) {
  int t = 0;
#pragma unroll
  for (int i = 1; i < MT; ++i) t += r >= i * cols;
  return t * tstride + xswz(r - t * cols);
}

template <bool Q4, int MT>
__device__ __forceinline__ void stage_word(const StagePlan &pp, float *dst, int f, uint64_t v) {
  // the word's elements lie in one op and one token row (each op's row is a
  // multiple of 64 elements) and land in one float4 slot
  const int e = (Q4 ? 2 : 4) * f;
  int k = pp.k0;
  while (k < pp.k1 && e >= (k + 1) * pp.epo) ++k;
  const int r = e - k * pp.epo;
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  float *od = dst + (k - pp.kbase) * pp.xstride;
  if constexpr (Q4)
    *(float2 *)(od + xq4(r)) = make_float2(__uint_as_float(lo), __uint_as_float(hi));
  else if constexpr (MT > 1)
    *(uint64_t *)((uint16_t *)od + x_pos<MT>(r, pp.epo / MT, 2 * pp.xstride / MT)) = v;
  else
    *(float4 *)(od + xswz(r)) =
        make_float4(bf16_to_f32(lo & 0xffffu), bf16_to_f32(lo >> 16), bf16_to_f32(hi & 0xffffu),
                    bf16_to_f32(hi >> 16));
}

// NB 64-bit words per lane of one op's input [base, wpo) into LDS: every
// load issued (clamped to the op's last word, never conditional) before any
// is consumed, so the whole batch costs one memory round trip.
template <bool Q4, int MT, int NB>
__device__ __forceinline__ void read_words(const uint64_t *op, float *od, int base, int wpo,
                                           int cols, int tstride, int lane) {
  uint64_t v[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) v[b] = ld_agent64(op + min(base + b * 64 + lane, wpo - 1));
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int f = base + b * 64 + lane;
    if (f < wpo) {
      const uint32_t lo = (uint32_t)v[b], hi = (uint32_t)(v[b] >> 32);
      if constexpr (Q4)
        *(float2 *)(od + xq4(2 * f)) = make_float2(__uint_as_float(lo), __uint_as_float(hi));
      else
        if constexpr (MT > 1)
          *(uint64_t *)((uint16_t *)od + x_pos<MT>(4 * f, cols, tstride)) = v[b];
        else
          *(float4 *)(od + xswz(4 * f)) =
              make_float4(__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u),
                          __uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u));
    }
  }
}

// A released stage input into LDS: agent-scope loads of the published
// words, then each lane's 64-bit words go to LDS as fp32.  Lane l takes
// words l, l + 64, ... of each op, so its LDS addresses advance by a
// constant: no per-element search.  The batch is sized to the op (one
// straight-line path per size, chosen before any load is issued): inputs
// up to 1536 words (a 3072-wide f32 row, a 6144-wide BF16 row) take one
// memory round trip, a 5120-wide f32 row two.
template <bool Q4, int MT>
__device__ void read_stage(const StagePlan &pp, float *dst, int lane) {
  const uint64_t *src = (const uint64_t *)pp.data;
  const int wpo = pp.epo >> (Q4 ? 1 : 2);  // 64-bit words per op (a multiple of 16)
  const int per_lane = uni((wpo + 63) >> 6);
  const int cols = pp.epo / MT, tstride = 2 * pp.xstride / MT;  // tstride: BF16 units
  for (int k = pp.k0; k <= pp.k1; ++k) {
    const uint64_t *op = src + (size_t)k * wpo;
    float *od = dst + (k - pp.kbase) * pp.xstride;
    if (per_lane <= 4)
      read_words<Q4, MT, 4>(op, od, 0, wpo, cols, tstride, lane);
    else if (per_lane <= 8)
      read_words<Q4, MT, 8>(op, od, 0, wpo, cols, tstride, lane);
    else if (per_lane <= 12)
      read_words<Q4, MT, 12>(op, od, 0, wpo, cols, tstride, lane);
    else
      for (int base = 0; base < wpo; base += 64 * 24)
        read_words<Q4, MT, 24>(op, od, base, wpo, cols, tstride, lane);
  }
}

// The first stage's input, straight from the ops' inputs (written before
// the launch).
template <bool Q4, int MT>
__device__ void read_first_stage(const StagePlan &pp, const StepOp *ops, const StepStage &st,
                                 float *dst, int lane) {
  constexpr int kEsz = Q4 ? 4 : 2;  // bytes per input element
  for (int f = pp.f0 + lane; f < pp.f1; f += 64) {
    const int e = (Q4 ? 2 : 4) * f, k = e / pp.epo;
    const QD_GLOBAL uint8_t *x = (const QD_GLOBAL uint8_t *)gp(ops[st.op0 + k].x);
    stage_word<Q4, MT>(pp, dst, f,
                       *(const QD_GLOBAL uint64_t *)(x + (size_t)(e - k * pp.epo) * kEsz));
  }
}

// Arrival at the barrier that releases stage s's input: after this
// workgroup's slice is stored (and acknowledged), one agent-scope atomic on
// its group's counter; the group's last arrival adds one to the stage's
// global counter, and the last of those writes the stage's tag into every
// workgroup's release line.  Counters only grow, so "last" is taken modulo
// the number of arrivals a launch makes.
__device__ __forceinline__ void arrive(uint32_t *ctr, uint32_t *rel, int s, uint32_t tag,
                                       int lane) {
  const int nwg = gridDim.x;
  const int g = blockIdx.x % kStepGroups;
  const unsigned gsz = (unsigned)((nwg - g + kStepGroups - 1) / kStepGroups);
  unsigned release = 0;
  if (lane == 0) {
    uint32_t *line = ctr + (size_t)(s * (kStepGroups + 1) + g) * kStepLine;
    const unsigned old = __hip_atomic_fetch_add(line, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if ((old + 1u) % gsz == 0u) {
      uint32_t *gl = ctr + (size_t)(s * (kStepGroups + 1) + kStepGroups) * kStepLine;
      const unsigned o2 = __hip_atomic_fetch_add(gl, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
      release = (o2 + 1u) % (unsigned)kStepGroups == 0u ? 1u : 0u;
    }
  }
  if (__builtin_amdgcn_readfirstlane(release))
    for (int k = lane; k < nwg; k += kWave) st_agent(rel + (size_t)k * kStepLine, tag);
}

template <bool Q4, int MT>
__device__ __forceinline__ void poller_wave(const StepOp *__restrict__ ops,
                                            const StepStage *__restrict__ stages,
                                            int n_stages, int m, Shared *sh, float *xbuf,
                                            int xmax, uint32_t *rel, uint32_t *ctr,
                                            uint32_t *err) {
  const int lane = threadIdx.x & 63;
  const uint32_t epoch = sh->epoch;
  const uint32_t *myrel = rel + (size_t)blockIdx.x * kStepLine;
  // after a first time-out this workgroup stops waiting, so a broken run
  // still ends quickly (with the error word set)
  bool aborted = false;
  // The values this workgroup publishes come from the resident inputs; they
  // are loaded kPubRing stages ahead into an LDS ring so that publishing is
  // an LDS read and a store, never a wait on memory.  Two stages suffice:
  // each load runs under a stage's compute.  (A 32-stage ring preloaded
  // before the first stage cost ~13 us per launch: 31 dependent load
  // chains before any compute wave could start.)
  PubSlice pending;
  int pending_stage = -1;
  StagePlan cur = stage_plan<Q4, MT>(ops, stages[0], m);
  StagePlan nxt = cur;
  for (int s = 0; s < n_stages; ++s) {
    const uint32_t tag = epoch + (uint32_t)s;
    // park the value loaded one stage ago (long since arrived)
    if (pending_stage >= 0) sh->pub[pending_stage % kPubRing][lane] = pending.v;
    if (s > 0 && !aborted) {
      unsigned polls = 0;
      while (__builtin_amdgcn_readfirstlane(ld_agent(myrel)) != tag) {
        if (++polls > kPollLimit) {
          if (lane == 0) atomicOr(err, 1u);
          aborted = true;
          break;
        }
      }
    }
    if (s == 0)
      read_first_stage<Q4, MT>(cur, ops, stages[0], xbuf, lane);
    else
      read_stage<Q4, MT>(cur, xbuf + (s & 1) * xmax, lane);
    if (kCompact<Q4, MT> && lane == 0) sh->xk0[s & 1] = cur.kbase;
    // hand the staged input to the compute waves (LDS executes this wave's
    // data writes before the flag write)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_store(&sh->xready, s + 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
    // resolve the next stage while the compute waves work
    if (s + 1 < n_stages) nxt = stage_plan<Q4, MT>(ops, stages[s + 1], m);
    // stage 1's values, needed at the end of this stage (later stages' come
    // through the ring below); loaded under stage 0's compute rather than
    // before the first input is staged
    if (s == 0 && n_stages > 1) {
      const PubSlice p = pub_load<Q4>(ops, stages[1], m, lane);
      sh->pub[1][lane] = p.v;
    }
    // load stage s + kPubRing's values; they are parked next iteration in the
    // slot of stage s, which was published at the end of the last iteration
    pending_stage = -1;
    if (s + kPubRing < n_stages) {
      pending = pub_load<Q4>(ops, stages[s + kPubRing], m, lane);
      pending_stage = s + kPubRing;
    }
    // wait for every compute wave to finish stage s, then publish s+1
    unsigned spins = 0;
    while (lds_ld(&sh->done) < (s + 1) * kNcw<Q4, MT>) {
      if (++spins > kLdsSpinLimit) {
        if (lane == 0) atomicOr(err, 2u);
        break;
      }
    }
    if (s + 1 < n_stages) {
      if (nxt.pa + lane < nxt.pb)
        st_agent(nxt.data + nxt.pa + lane, sh->pub[(s + 1) % kPubRing][lane]);
      // the slice is acknowledged (visible device-wide) before the arrival
      // that may release it
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      arrive(ctr, rel, s + 1, tag + 1u, lane);
      // the compute waves may now issue the next stage's weights
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (lane == 0) __hip_atomic_store(&sh->arrived, s + 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    cur = nxt;
  }
}

template <bool Q4, int MT, int NG>
__device__ __forceinline__ void step_body(const StepOp *__restrict__ ops,
                                          const StepStage *__restrict__ stages, int n_stages,
                                          int m, int xmax, int nwg, uint32_t *epoch_word,
                                          uint32_t *rel, uint32_t *ctr, uint32_t *err) {
  if ((int)gridDim.x != nwg) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err, 8u);
    return;
  }
  __shared__ Shared sh;
  extern __shared__ __attribute__((aligned(16))) float xbuf[];  // [2][xmax]
  if (threadIdx.x == 0) {
    sh.xready = 0;
    sh.done = 0;
    sh.arrived = 0;
    sh.epoch = ld_agent(epoch_word);
    sh.xk0[0] = sh.xk0[1] = 0;
  }
  __syncthreads();
  if (threadIdx.x < kWave)
    poller_wave<Q4, MT>(ops, stages, n_stages, m, &sh, xbuf, xmax, rel, ctr, err);
  else
    compute_wave<Q4, MT, NG>(ops, stages, n_stages, &sh, xbuf, xmax, err);
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0) st_agent(epoch_word, sh.epoch + (uint32_t)n_stages);
}

template <int NG>
__global__ __launch_bounds__((kThreads<false, 1>)) void affine_step_kernel(
    const StepOp *__restrict__ ops, const StepStage *__restrict__ stages, int n_stages,
    int m, int xmax, int nwg, uint32_t *__restrict__ epoch_word, uint32_t *__restrict__ rel,
    uint32_t *__restrict__ ctr, uint32_t *__restrict__ err) {
  step_body<false, 1, NG>(ops, stages, n_stages, m, xmax, nwg, epoch_word, rel, ctr, err);
}

// m = MT token rows (2..4) of affine ops
template <int MT>
__global__ __launch_bounds__((kThreads<false, MT>)) void affine_step_mt_kernel(
    const StepOp *__restrict__ ops, const StepStage *__restrict__ stages, int n_stages,
    int m, int xmax, int nwg, uint32_t *__restrict__ epoch_word, uint32_t *__restrict__ rel,
    uint32_t *__restrict__ ctr, uint32_t *__restrict__ err) {
  step_body<false, MT, kGroupItems>(ops, stages, n_stages, m, xmax, nwg, epoch_word, rel, ctr,
                                    err);
}

__global__ __launch_bounds__((kThreads<true, 1>)) void q4_0_step_kernel(
    const StepOp *__restrict__ ops, const StepStage *__restrict__ stages, int n_stages,
    int m, int xmax, int nwg, uint32_t *__restrict__ epoch_word, uint32_t *__restrict__ rel,
    uint32_t *__restrict__ ctr, uint32_t *__restrict__ err) {
  step_body<true, 1, kGroupItems>(ops, stages, n_stages, m, xmax, nwg, epoch_word, rel, ctr,
                                  err);
}

}  // namespace

int step_compute_waves(bool q4, int m) {
  return q4 ? kNcw<true, 1> : m > 1 ? kNcw<false, 2> : kNcw<false, 1>;
}

bool step_compact(bool q4, int m) { return q4 ? kCompact<true, 1> : kCompact<false, 2> && m > 1; }

hipError_t launch_step(bool q4, const StepOp *ops, const StepStage *stages, int n_stages, int m,
                       int xmax, int nwg, uint32_t *epoch_word, uint32_t *rel, uint32_t *ctr,
                       uint32_t *err, size_t lds_bytes, int group, hipStream_t stream) {
  const void *fn;
  int threads;
  if (q4) {
    fn = (const void *)q4_0_step_kernel;
    threads = kThreads<true, 1>;
  } else if (m == 1) {
    fn = group == 4 ? (const void *)affine_step_kernel<4>
                    : (const void *)affine_step_kernel<kGroupItems>;
    threads = kThreads<false, 1>;
  } else if (m == 2) {
    fn = (const void *)affine_step_mt_kernel<2>;
    threads = kThreads<false, 2>;
  } else if (m == 3) {
    fn = (const void *)affine_step_mt_kernel<3>;
    threads = kThreads<false, 3>;
  } else if (m == 4) {
    fn = (const void *)affine_step_mt_kernel<4>;
    threads = kThreads<false, 4>;
  } else {
    return hipErrorInvalidValue;
  }
  if (lds_bytes > 65536) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds_bytes);
    if (e != hipSuccess) return e;
  }
  void *args[] = {(void *)&ops,  (void *)&stages,     (void *)&n_stages, (void *)&m,
                  (void *)&xmax, (void *)&nwg,        (void *)&epoch_word, (void *)&rel,
                  (void *)&ctr,  (void *)&err};
  hipError_t e = hipLaunchKernel(fn, dim3(nwg), dim3(threads), args, lds_bytes, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace qd
