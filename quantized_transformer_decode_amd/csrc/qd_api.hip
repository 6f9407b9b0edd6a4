// qd_api.hip -- the extern "C" entry points of libqdecode.so (include/qdecode.h).
//
// Every argument is checked on the host before the first HIP call, so a host
// without a GPU can exercise every error path.  Only then is the current
// device checked (gfx950, cached per device) and the kernels enqueued on the
// caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <cmath>

#include "../../include/qdecode.h"
#include "qd_internal.h"
#include "qd_step.h"

#include <vector>

namespace {

constexpr int64_t kMaxGemvCols = 8192;  // LDS copy of x per workgroup
constexpr int64_t kMaxGemmCols = 65536;
constexpr int64_t kMaxGemmM = int64_t(1) << 22;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

thread_local int g_last_hip = 0;

// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_arch[64];

std::atomic<int> g_cus[64];

// Compute units of the current device (0 on failure).
int current_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev < 64) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (dev < 64) g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

qd_status hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return QD_EHIP;
}

qd_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return QD_EDEVICE;
  }
  if (dev < 64) {
    const int c = g_arch[dev].load(std::memory_order_relaxed);
    if (c == 1) return QD_OK;
    if (c == 2) return QD_EDEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return QD_EDEVICE;
  }
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_arch[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? QD_OK : QD_EDEVICE;
}

size_t affine_bytes(int64_t rows, int64_t cols) {
  return (size_t)rows * cols + 2 * (size_t)rows * (cols / 64) * 2;
}

size_t q40_bytes(int64_t rows, int64_t cols) {
  const size_t total = (size_t)rows * (cols / 32) * 18;
  return (total + 3) & ~(size_t)3;
}

bool affine_shape_ok(int64_t rows, int64_t cols) {
  return rows >= 1 && cols >= 64 && cols % 64 == 0;
}

constexpr int kMaxStageWords = 16384;  // LDS: two fp32 copies of a stage input
constexpr int kMinStepWgs = 32;        // smallest grid a plan supports
constexpr int kMaxStepRows = 4;        // token rows of an affine step
// a last stage of one GEMV of at least this many weights runs as its own launch
constexpr int64_t kStepTailWeights = (int64_t)1 << 27;
// log2 of the slice length for a stage input of `words` 32-bit words over
// `nwg` publishers: the smallest power of two >= ceil(words / nwg), within
// [1, 64] words (one per lane of the publishing wave).
int step_lg(int64_t words, int nwg) {
  const int64_t per = (words + nwg - 1) / nwg;
  int lg = 1;
  while ((int64_t(1) << lg) < per) ++lg;
  return lg;
}
constexpr int64_t kMaxStepOps = 65536;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// One GEMV of a decode step, either format (the public op structs differ
// only in their pointer types).
struct StepIn {
  const void *w, *x;
  void *y;
  int64_t rows, cols, stage;
};

// What the two formats' step plans differ in.
struct StepFormat {
  bool q4;
  int elem() const { return q4 ? 4 : 2; }        // bytes per input / output element
  int chunk() const { return q4 ? 2048 : 1024; } // columns per work item
  int per_word() const { return q4 ? 1 : 2; }    // input values per 32-bit exchange word
  size_t weights(int64_t rows, int64_t cols) const {
    return q4 ? q40_bytes(rows, cols) : affine_bytes(rows, cols);
  }
  bool cols_ok(int64_t cols) const {
    return q4 ? cols % 256 == 0 && cols >= 256 && cols <= kMaxGemvCols
              : cols % 64 == 0 && cols <= kMaxGemvCols;
  }
};

std::vector<StepIn> step_in(const qd_affine_gemv_op *ops, int64_t n_ops) {
  std::vector<StepIn> v((size_t)n_ops);
  for (int64_t i = 0; i < n_ops; ++i)
    v[i] = StepIn{ops[i].w_packed, ops[i].x_bf16, ops[i].y_bf16, ops[i].rows, ops[i].cols,
                  ops[i].stage};
  return v;
}
std::vector<StepIn> step_in(const qd_q4_0_gemv_op *ops, int64_t n_ops) {
  std::vector<StepIn> v((size_t)n_ops);
  for (int64_t i = 0; i < n_ops; ++i)
    v[i] = StepIn{ops[i].w_q4_0, ops[i].x, ops[i].y, ops[i].rows, ops[i].cols, ops[i].stage};
  return v;
}

// LDS floats one op's staged input takes: whole chunks of the item width,
// fp32 for one token row, BF16 (half a float each) for several.
int64_t step_op_lds_floats(int64_t cols, int64_t m, StepFormat f) {
  const int64_t items = (cols + f.chunk() - 1) / f.chunk() * f.chunk();
  return m == 1 ? items : m * items / 2;
}

// Validates a decode-step op list; on success fills the layout sizes.
qd_status step_validate(const StepIn *ops, int64_t n_ops, int64_t m, StepFormat f,
                        size_t *ws_bytes, int *n_stages) {
  // several token rows for affine ops (one persistent kernel per row count)
  if (!ops || n_ops < 1 || n_ops > kMaxStepOps || m < 1 || m > (f.q4 ? 1 : kMaxStepRows))
    return QD_EINVAL;
  int stages = 0;
  for (int64_t i = 0; i < n_ops; ++i) {
    const StepIn &o = ops[i];
    if (!o.w || !o.x || !o.y) return QD_EINVAL;
    if (o.rows < 1 || o.rows > kMaxRows || o.cols < 1) return QD_EINVAL;
    if (!f.cols_ok(o.cols)) return QD_ESHAPE;
    if (!aligned(o.w, 16) || !aligned(o.x, 16) || !aligned(o.y, f.elem())) return QD_EALIGN;
    if (i == 0) {
      if (o.stage != 0) return QD_EINVAL;
      stages = 1;
    } else if (o.stage == ops[i - 1].stage + 1) {
      stages += 1;
    } else if (o.stage == ops[i - 1].stage) {
      if (o.cols != ops[i - 1].cols) return QD_ESHAPE;
    } else {
      return QD_EINVAL;
    }
    // LDS holds an op's input in whole chunks of the format's item width
    if (step_op_lds_floats(o.cols, m, f) > kMaxStageWords) return QD_ESHAPE;
  }
  // outputs may not overlap any weights or inputs of the step
  for (int64_t i = 0; i < n_ops; ++i) {
    const size_t ny = (size_t)m * ops[i].rows * f.elem();
    for (int64_t j = 0; j < n_ops; ++j) {
      if (overlap(ops[i].y, ny, ops[j].w, f.weights(ops[j].rows, ops[j].cols)) ||
          overlap(ops[i].y, ny, ops[j].x, (size_t)m * ops[j].cols * f.elem()))
        return QD_EINVAL;
      if (j > i && overlap(ops[i].y, ny, ops[j].y, (size_t)m * ops[j].rows * f.elem()))
        return QD_EINVAL;
    }
  }
  *n_stages = stages;
  *ws_bytes = sizeof(qd::StepHeader) + align256(sizeof(qd::StepOp) * n_ops) +
              align256(sizeof(qd::StepStage) * stages);
  return QD_OK;
}

// Each workgroup publishes at most 64 words of a stage's input, one per
// lane: at most 128 BF16 values (affine) or 64 f32 values (Q4_0) per
// workgroup.
bool step_fits_grid(const StepIn *ops, int64_t n_ops, int64_t m, int nwg, StepFormat f) {
  int64_t i = 0;
  while (i < n_ops) {
    int64_t j = i, values = 0;
    while (j < n_ops && ops[j].stage == ops[i].stage) values += m * ops[j++].cols;
    if (values > (int64_t)64 * f.per_word() * nwg) return false;
    i = j;
  }
  return true;
}

// fp32 LDS floats one staged stage input takes at most in a workgroup: with
// several token rows the ops its rows fall in (the kernel splits each
// stage's rows evenly over all compute waves, workgroup j holding those of
// its waves), else every op of the stage; m token rows of whole items each.
// 0 if some workgroup would need more than the LDS holds.
int step_lds_floats(const StepIn *ops, int64_t n_ops, int64_t m, int nwg, StepFormat f) {
  const int64_t ncw = qd::step_compute_waves(f.q4, (int)m);
  const int64_t nw = (int64_t)nwg * ncw;
  int64_t worst = 0;
  int64_t i = 0;
  while (i < n_ops) {
    int64_t j = i, total = 0;
    while (j < n_ops && ops[j].stage == ops[i].stage) total += ops[j++].rows;
    const int64_t per_op = step_op_lds_floats(ops[i].cols, m, f);
    for (int64_t g = 0; g < nwg; ++g) {
      const int64_t lo = total * (g * ncw) / nw, hi = total * ((g + 1) * ncw) / nw;
      if (hi <= lo) continue;
      // ops holding rows lo and hi - 1 of the stage's row space
      int64_t k0 = -1, k1 = -1, base = 0;
      for (int64_t k = i; k < j; ++k) {
        if (k0 < 0 && lo < base + ops[k].rows) k0 = k;
        if (k1 < 0 && hi - 1 < base + ops[k].rows) k1 = k;
        base += ops[k].rows;
      }
      const int64_t need = (qd::step_compact(f.q4, (int)m) ? k1 - k0 + 1 : j - i) * per_op;
      if (need > worst) worst = need;
    }
    i = j;
  }
  return worst > kMaxStageWords ? 0 : (int)worst;
}

// Bytes after the tables: one release line per workgroup, the arrival
// counter lines, and each stage's dense input (256-byte aligned).
size_t step_exchange_bytes(const StepIn *ops, int64_t n_ops, int64_t m, int nwg, int n_stages,
                           StepFormat f) {
  size_t bytes = align256((size_t)nwg * 128) +
                 align256((size_t)n_stages * (qd::kStepGroups + 1) * 128);
  int64_t i = 0;
  while (i < n_ops) {
    int64_t j = i, values = 0;
    while (j < n_ops && ops[j].stage == ops[i].stage) values += m * ops[j++].cols;
    bytes += align256((size_t)values * f.elem());
    i = j;
  }
  return bytes;
}

size_t step_workspace_bytes(const StepIn *ops, int64_t n_ops, int64_t m, StepFormat f) {
  size_t bytes = 0;
  int ns = 0;
  if (step_validate(ops, n_ops, m, f, &bytes, &ns) != QD_OK) return 0;
  // the staging layout depends on the grid: one workgroup per CU of the
  // current device
  if (check_device() != QD_OK) return 0;
  const int nwg = current_cus();
  if (nwg < kMinStepWgs || !step_fits_grid(ops, n_ops, m, nwg, f)) return 0;
  if (step_lds_floats(ops, n_ops, m, nwg, f) == 0) return 0;
  return bytes + step_exchange_bytes(ops, n_ops, m, nwg, ns, f);
}

qd_status step_plan(const StepIn *ops, int64_t n_ops, int64_t m, StepFormat f, void *workspace,
                    size_t workspace_bytes, qd_step_plan *plan, void *stream) {
  if (!workspace || !plan) return QD_EINVAL;
  size_t need = 0;
  int ns = 0;
  qd_status st = step_validate(ops, n_ops, m, f, &need, &ns);
  if (st != QD_OK) return st;
  if (!aligned(workspace, 256)) return QD_EALIGN;
  if (workspace_bytes < need) return QD_EINVAL;  // tables alone; staging checked below
  for (int64_t i = 0; i < n_ops; ++i) {
    const StepIn &o = ops[i];
    if (overlap(workspace, workspace_bytes, o.w, f.weights(o.rows, o.cols)) ||
        overlap(workspace, workspace_bytes, o.x, (size_t)m * o.cols * f.elem()) ||
        overlap(workspace, workspace_bytes, o.y, (size_t)m * o.rows * f.elem()))
      return QD_EINVAL;
  }
  st = check_device();
  if (st != QD_OK) return st;
  const int nwg = current_cus();
  if (nwg < kMinStepWgs) return QD_EDEVICE;
  if (!step_fits_grid(ops, n_ops, m, nwg, f)) return QD_ESHAPE;
  const int xmax = step_lds_floats(ops, n_ops, m, nwg, f);
  if (xmax == 0) return QD_ESHAPE;
  need += step_exchange_bytes(ops, n_ops, m, nwg, ns, f);
  if (workspace_bytes < need) return QD_EINVAL;

  // host image of header + tables; release lines and counters start zeroed
  // (tag 0 is never expected: the epoch starts at 1)
  const size_t ops_off = sizeof(qd::StepHeader);
  const size_t stages_off = ops_off + align256(sizeof(qd::StepOp) * n_ops);
  const size_t rel_off = stages_off + align256(sizeof(qd::StepStage) * ns);
  const size_t ctr_off = rel_off + align256((size_t)nwg * 128);
  const size_t data_off = ctr_off + align256((size_t)ns * (qd::kStepGroups + 1) * 128);
  const size_t stg_off = rel_off;
  std::vector<uint8_t> img(rel_off, 0);
  qd::StepHeader *h = (qd::StepHeader *)img.data();
  qd::StepOp *dops = (qd::StepOp *)(img.data() + ops_off);
  qd::StepStage *dst = (qd::StepStage *)(img.data() + stages_off);
  h->magic = qd::kStepMagic;
  h->n_ops = (int32_t)n_ops;
  h->n_stages = ns;
  h->m = (int32_t)m;
  h->nwg = nwg;
  h->xmax = xmax;
  h->ops_off = (uint32_t)ops_off;
  h->stages_off = (uint32_t)stages_off;
  h->rel_off = (uint32_t)rel_off;
  h->ctr_off = (uint32_t)ctr_off;
  h->data_off = (uint32_t)data_off;
  h->lds_bytes = (uint32_t)(2 * (size_t)xmax * 4);
  h->epoch = 1;
  h->error = 0;
  size_t data = data_off;
  int s = -1;
  for (int64_t i = 0; i < n_ops; ++i) {
    const StepIn &o = ops[i];
    if ((int)o.stage != s) {
      s = (int)o.stage;
      int64_t values = 0;
      for (int64_t j = i; j < n_ops && ops[j].stage == o.stage; ++j) values += m * ops[j].cols;
      const int64_t words = values / f.per_word();
      dst[s].data = (uint32_t *)((uint8_t *)workspace + data);
      dst[s].op0 = (int32_t)i;
      dst[s].nops = 0;
      dst[s].rows_total = 0;
      dst[s].cols = (int32_t)o.cols;
      dst[s].chunks = (int32_t)((o.cols + f.chunk() - 1) / f.chunk());
      dst[s].words = (uint16_t)words;
      dst[s].lg = (uint16_t)step_lg(words, nwg);
      data += align256((size_t)values * f.elem());
    }
    qd::StepOp &d = dops[i];
    d.w = (const uint8_t *)o.w;
    d.x = (const uint16_t *)o.x;
    d.y = (uint16_t *)o.y;
    d.unused = nullptr;
    d.rows = (int32_t)o.rows;
    d.cols = (int32_t)o.cols;
    d.stage = s;
    d.row_base = dst[s].rows_total;
    dst[s].rows_total += (int32_t)o.rows;
    dst[s].nops += 1;
  }
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(workspace, img.data(), img.size(), hipMemcpyHostToDevice, hs);
  if (e == hipSuccess)
    e = hipMemsetAsync((uint8_t *)workspace + stg_off, 0, need - stg_off, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return hip_fail(e);
  plan->workspace = workspace;
  plan->nwg = nwg;
  plan->lds_bytes = (int32_t)h->lds_bytes;
  plan->n_ops = (int32_t)n_ops;
  plan->n_stages = ns;
  plan->m = (int32_t)m;
  plan->magic = qd::kStepMagic;
  plan->format = f.q4 ? 1 : 0;
  // register groups of four items for a single-row affine plan whose stages
  // give each compute wave more than three items on average (the persistent
  // kernel's stages: the tail, when streamed on its own, does not count)
  {
    const int64_t nw = (int64_t)nwg * qd::step_compute_waves(f.q4, (int)m);
    const int last = ns - ((!f.q4 && ns > 1 && (n_ops == 1 || ops[n_ops - 2].stage !=
                                                ops[n_ops - 1].stage) &&
                            ops[n_ops - 1].rows * ops[n_ops - 1].cols >= kStepTailWeights)
                               ? 1 : 0);
    int64_t items = 0;
    for (int64_t i = 0; i < n_ops; ++i)
      if (ops[i].stage < last) items += ops[i].rows * ((ops[i].cols + f.chunk() - 1) / f.chunk());
    plan->group = (!f.q4 && m == 1 && last > 0 && items > 3 * nw * (int64_t)last) ? 4 : 3;
  }
  // a last stage of one very large affine GEMV streams faster as its own
  // launch
  const StepIn &last = ops[n_ops - 1];
  const bool tail = !f.q4 && ns > 1 && (n_ops == 1 || ops[n_ops - 2].stage != last.stage) &&
                    last.rows * last.cols >= kStepTailWeights;
  plan->tail = tail ? 1 : 0;
  plan->tail_w = tail ? last.w : nullptr;
  plan->tail_x = tail ? last.x : nullptr;
  plan->tail_y = tail ? last.y : nullptr;
  plan->tail_rows = tail ? last.rows : 0;
  plan->tail_cols = tail ? last.cols : 0;
  return QD_OK;
}

qd_status step_run(const qd_step_plan *plan, bool q4, void *stream) {
  if (!plan || !plan->workspace || plan->magic != qd::kStepMagic ||
      plan->format != (q4 ? 1 : 0) || plan->nwg < 1 || plan->lds_bytes < 8 ||
      plan->lds_bytes > 2 * kMaxStageWords * 4 || plan->lds_bytes % 8 != 0 ||
      plan->n_ops < 1 || plan->n_stages < 1 || plan->n_stages > plan->n_ops ||
      plan->m < 1 || plan->m > (q4 ? 1 : kMaxStepRows) || plan->tail < 0 || plan->tail > 1 ||
      (q4 && plan->tail) ||
      (plan->tail && (plan->n_stages < 2 || !plan->tail_w || !plan->tail_x || !plan->tail_y ||
                      plan->tail_rows < 1 || plan->tail_cols < 64 || plan->tail_cols % 64 ||
                      plan->tail_cols > kMaxGemvCols)))
    return QD_EINVAL;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  if (current_cus() != plan->nwg) return QD_EDEVICE;
  uint8_t *ws = (uint8_t *)plan->workspace;
  const size_t ops_off = sizeof(qd::StepHeader);
  const size_t stages_off = ops_off + align256(sizeof(qd::StepOp) * plan->n_ops);
  qd::StepHeader *h = (qd::StepHeader *)ws;  // device address; never dereferenced here
  const size_t rel_off = stages_off + align256(sizeof(qd::StepStage) * plan->n_stages);
  const size_t ctr_off = rel_off + align256((size_t)plan->nwg * 128);
  hipError_t e = qd::launch_step(
      q4, (const qd::StepOp *)(ws + ops_off), (const qd::StepStage *)(ws + stages_off),
      plan->n_stages - plan->tail, plan->m, plan->lds_bytes / 8, plan->nwg, &h->epoch,
      (uint32_t *)(ws + rel_off), (uint32_t *)(ws + ctr_off), &h->error,
      (size_t)plan->lds_bytes, plan->group, (hipStream_t)stream);
  if (e == hipSuccess && plan->tail) {
    qd::AffineGroup g = {};
    g.n = 1;
    g.w[0] = (const uint8_t *)plan->tail_w;
    g.y[0] = (uint16_t *)plan->tail_y;
    g.rows[0] = (int)plan->tail_rows;
    e = qd::launch_affine_gemv(g, (int)plan->tail_cols, (const uint16_t *)plan->tail_x, plan->m,
                               false, (hipStream_t)stream);
  }
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

qd_status step_check(const qd_step_plan *plan, bool q4, uint32_t *error_bits, void *stream) {
  if (!plan || !plan->workspace || plan->magic != qd::kStepMagic ||
      plan->format != (q4 ? 1 : 0) || !error_bits)
    return QD_EINVAL;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  uint32_t v = 0;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(&v, (uint8_t *)plan->workspace + offsetof(qd::StepHeader, error),
                                4, hipMemcpyDeviceToHost, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return hip_fail(e);
  *error_bits = v;
  return v ? QD_ESTEP : QD_OK;
}

}  // namespace

int qd::device_cus() { return current_cus(); }

extern "C" {

const char *qd_status_string(int status) {
  switch (status) {
    case QD_OK: return "QD_OK";
    case QD_EINVAL: return "QD_EINVAL: invalid argument (null pointer, size out of range or overlapping buffers)";
    case QD_ESHAPE: return "QD_ESHAPE: matrix width violates the format's divisibility rule";
    case QD_EALIGN: return "QD_EALIGN: pointer not aligned as the kernel requires";
    case QD_EDEVICE: return "QD_EDEVICE: no current HIP device, or it is not gfx950";
    case QD_EHIP: return "QD_EHIP: the HIP runtime reported an error";
    case QD_ESTEP: return "QD_ESTEP: a decode-step launch reported a wait time-out or grid mismatch";
    case QD_ESCRATCH: return "QD_ESCRATCH: the shape needs more than the library's static scratch buffer";
    default: return "QD_UNKNOWN";
  }
}

int qd_last_hip_error(void) { return g_last_hip; }

const char *qd_version(void) { return "qdecode 0.1.0 gfx950"; }

size_t affine_i8_g64_bytes(int64_t rows, int64_t cols) {
  return affine_shape_ok(rows, cols) ? affine_bytes(rows, cols) : 0;
}

size_t affine_i8_g64_scales_offset(int64_t rows, int64_t cols) {
  return affine_shape_ok(rows, cols) ? (size_t)rows * cols : 0;
}

size_t affine_i8_g64_biases_offset(int64_t rows, int64_t cols) {
  return affine_shape_ok(rows, cols)
             ? (size_t)rows * cols + (size_t)rows * (cols / 64) * 2
             : 0;
}

size_t q4_0_bytes(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 32 || cols % 32 != 0) return 0;
  return q40_bytes(rows, cols);
}

qd_status affine_i8_g64_pack(const void *codes_u32, const void *scales_bf16,
                             const void *biases_bf16, int64_t rows,
                             int64_t cols, void *blob, void *stream) {
  if (!codes_u32 || !scales_bf16 || !biases_bf16 || !blob) return QD_EINVAL;
  if (rows < 1 || rows > kMaxRows || cols < 1) return QD_EINVAL;
  if (cols % 64 != 0) return QD_ESHAPE;
  if (!aligned(blob, 16)) return QD_EALIGN;
  const size_t nc = (size_t)rows * cols;
  const size_t ns = (size_t)rows * (cols / 64) * 2;
  const size_t nt = affine_bytes(rows, cols);
  if (overlap(blob, nt, codes_u32, nc) || overlap(blob, nt, scales_bf16, ns) ||
      overlap(blob, nt, biases_bf16, ns))
    return QD_EINVAL;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *dst = (uint8_t *)blob;
  hipError_t e = hipMemcpyAsync(dst, codes_u32, nc, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dst + nc, scales_bf16, ns, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dst + nc + ns, biases_bf16, ns, hipMemcpyDeviceToDevice, s);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

}  // extern "C"

// The affine GEMVs of one launch (shared input x), activations BF16 or f16.
static qd_status affine_group(const qd_affine_gemv_item *items, int64_t n_items, int64_t cols,
                              const void *x_bf16, int64_t m, bool f16, void *stream) {
  if (!items || !x_bf16 || n_items < 1 || n_items > qd::kMaxGroup) return QD_EINVAL;
  if (m < 1 || m > 16 || cols < 1) return QD_EINVAL;
  if (cols % 64 != 0 || cols > kMaxGemvCols) return QD_ESHAPE;
  if (!aligned(x_bf16, 16)) return QD_EALIGN;
  for (int64_t k = 0; k < n_items; ++k) {
    const qd_affine_gemv_item &it = items[k];
    if (!it.w_packed || !it.y_bf16) return QD_EINVAL;
    if (it.rows < 1 || it.rows > kMaxRows) return QD_EINVAL;
    if (!aligned(it.w_packed, 16) || !aligned(it.y_bf16, 2)) return QD_EALIGN;
  }
  // an output may overlap neither the input, nor any weights, nor another output
  for (int64_t k = 0; k < n_items; ++k) {
    const size_t ny = (size_t)m * items[k].rows * 2;
    if (overlap(items[k].y_bf16, ny, x_bf16, (size_t)m * cols * 2)) return QD_EINVAL;
    for (int64_t j = 0; j < n_items; ++j) {
      if (overlap(items[k].y_bf16, ny, items[j].w_packed, affine_bytes(items[j].rows, cols)))
        return QD_EINVAL;
      if (j > k && overlap(items[k].y_bf16, ny, items[j].y_bf16, (size_t)m * items[j].rows * 2))
        return QD_EINVAL;
    }
  }
  qd_status st = check_device();
  if (st != QD_OK) return st;
  qd::AffineGroup g = {};
  g.n = (int)n_items;
  for (int64_t k = 0; k < n_items; ++k) {
    g.w[k] = (const uint8_t *)items[k].w_packed;
    g.y[k] = (uint16_t *)items[k].y_bf16;
    g.rows[k] = (int)items[k].rows;
  }
  hipError_t e = qd::launch_affine_gemv(g, (int)cols, (const uint16_t *)x_bf16, (int)m, f16,
                                        (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

extern "C" {

qd_status qgemv_affine_i8_g64(const void *w_packed, int64_t rows, int64_t cols,
                              const void *x_bf16, void *y_bf16, int64_t m,
                              void *stream) {
  const qd_affine_gemv_item item = {w_packed, y_bf16, rows};
  return affine_group(&item, 1, cols, x_bf16, m, false, stream);
}

qd_status qgemv_affine_i8_g64_group(const qd_affine_gemv_item *items, int64_t n_items,
                                    int64_t cols, const void *x_bf16, int64_t m,
                                    void *stream) {
  return affine_group(items, n_items, cols, x_bf16, m, false, stream);
}

qd_status qgemv_affine_i8_g64_f16(const void *w_packed, int64_t rows, int64_t cols,
                                  const void *x_f16, void *y_f16, int64_t m, void *stream) {
  const qd_affine_gemv_item item = {w_packed, y_f16, rows};
  return affine_group(&item, 1, cols, x_f16, m, true, stream);
}

qd_status affine_i8_g64_embed_rows(const void *w_packed, int64_t rows, int64_t cols,
                                   const int64_t *token_ids, int64_t n, void *out,
                                   int32_t out_f16, void *stream) {
  if (!w_packed || !token_ids || !out) return QD_EINVAL;
  if (n < 1 || n > qd::kMaxEmbedTokens || (out_f16 != 0 && out_f16 != 1)) return QD_EINVAL;
  if (rows < 1 || rows > kMaxRows || cols < 1) return QD_EINVAL;
  if (cols % 64 != 0 || cols > kMaxGemvCols) return QD_ESHAPE;
  if (!aligned(w_packed, 16) || !aligned(out, 8)) return QD_EALIGN;
  qd::EmbedTokens tk = {};
  tk.n = (int)n;
  for (int64_t i = 0; i < n; ++i) {
    if (token_ids[i] < 0 || token_ids[i] >= rows) return QD_EINVAL;
    tk.t[i] = (int)token_ids[i];
  }
  if (overlap(out, (size_t)n * cols * 2, w_packed, affine_bytes(rows, cols))) return QD_EINVAL;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = qd::launch_affine_embed_rows((const uint8_t *)w_packed, (int)rows, (int)cols,
                                              tk, (uint16_t *)out, out_f16 == 1,
                                              (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

}  // extern "C"

// q_linear products of one launch (shared input): validation shared by the
// GEMV (f32 x, m <= 16) and the GEMM (BF16 x, any m) forms.
static qd_status q40_linear_check(const qd_q4_0_linear_item *items, int64_t n_items,
                                  int64_t cols, const void *x, size_t xbytes, int64_t m,
                                  int32_t gelu, size_t y_align) {
  if (!items || !x || n_items < 1 || n_items > qd::kMaxGroup) return QD_EINVAL;
  if (gelu != 0 && gelu != 1) return QD_EINVAL;
  if (!aligned(x, 16)) return QD_EALIGN;
  for (int64_t k = 0; k < n_items; ++k) {
    const qd_q4_0_linear_item &it = items[k];
    if (!it.w_q4_0 || !it.y) return QD_EINVAL;
    if (it.rows < 1 || it.rows > kMaxRows) return QD_EINVAL;
    if (!aligned(it.w_q4_0, 16) || !aligned(it.y, y_align) || !aligned(it.bias, 4))
      return QD_EALIGN;
  }
  // an output may overlap neither the input, nor any weights or bias, nor
  // another output
  for (int64_t k = 0; k < n_items; ++k) {
    const size_t ny = (size_t)m * items[k].rows * 4;
    if (overlap(items[k].y, ny, x, xbytes)) return QD_EINVAL;
    for (int64_t j = 0; j < n_items; ++j) {
      if (overlap(items[k].y, ny, items[j].w_q4_0, q40_bytes(items[j].rows, cols)) ||
          (items[j].bias && overlap(items[k].y, ny, items[j].bias, (size_t)items[j].rows * 4)))
        return QD_EINVAL;
      if (j > k && overlap(items[k].y, ny, items[j].y, (size_t)m * items[j].rows * 4))
        return QD_EINVAL;
    }
  }
  return QD_OK;
}

static qd::Q40Group q40_group(const qd_q4_0_linear_item *items, int64_t n_items, int32_t gelu) {
  qd::Q40Group g = {};
  g.n = (int)n_items;
  g.gelu = gelu;
  for (int64_t k = 0; k < n_items; ++k) {
    g.w[k] = (const uint8_t *)items[k].w_q4_0;
    g.y[k] = items[k].y;
    g.bias[k] = items[k].bias;
    g.rows[k] = (int)items[k].rows;
  }
  return g;
}

extern "C" {

qd_status qlinear_q4_0_gemv(const qd_q4_0_linear_item *items, int64_t n_items, int64_t cols,
                            const float *x, int64_t m, int32_t gelu, void *stream) {
  if (m < 1 || m > 16 || cols < 1) return QD_EINVAL;
  if (cols % 256 != 0 || cols > kMaxGemvCols) return QD_ESHAPE;
  qd_status st = q40_linear_check(items, n_items, cols, x, (size_t)m * cols * 4, m, gelu, 4);
  if (st != QD_OK) return st;
  st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = qd::launch_q4_0_gemv(q40_group(items, n_items, gelu), (int)cols, x, (int)m,
                                      (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

qd_status qlinear_q4_0_gemm(const qd_q4_0_linear_item *items, int64_t n_items, int64_t cols,
                            const void *x_bf16, int64_t m, int32_t gelu, void *stream) {
  if (m < 1 || m > kMaxGemmM || cols < 1) return QD_EINVAL;
  if (cols % 256 != 0 || cols > kMaxGemmCols) return QD_ESHAPE;
  qd_status st = q40_linear_check(items, n_items, cols, x_bf16, (size_t)m * cols * 2, m, gelu,
                                  16);
  if (st != QD_OK) return st;
  st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = qd::launch_q4_0_gemm(q40_group(items, n_items, gelu), (int)cols,
                                      (const uint16_t *)x_bf16, (int)m, (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

qd_status qgemv_q4_0(const void *w_q4_0, int64_t rows, int64_t cols,
                     const float *x, float *y, int64_t m, void *stream) {
  const qd_q4_0_linear_item item = {w_q4_0, nullptr, y, rows};
  return qlinear_q4_0_gemv(&item, 1, cols, x, m, 0, stream);
}

qd_status qgemv_q4_0_group(const qd_q4_0_gemv_item *items, int64_t n_items, int64_t cols,
                           const float *x, int64_t m, void *stream) {
  if (!items || n_items < 1 || n_items > qd::kMaxGroup) return QD_EINVAL;
  qd_q4_0_linear_item li[qd::kMaxGroup];
  for (int64_t k = 0; k < n_items; ++k) li[k] = {items[k].w_q4_0, nullptr, items[k].y, items[k].rows};
  return qlinear_q4_0_gemv(li, n_items, cols, x, m, 0, stream);
}

qd_status qgemm_q4_0_prefill(const void *w_q4_0, int64_t rows, int64_t cols,
                             const void *x_bf16, float *y, int64_t m,
                             void *stream) {
  const qd_q4_0_linear_item item = {w_q4_0, nullptr, y, rows};
  return qlinear_q4_0_gemm(&item, 1, cols, x_bf16, m, 0, stream);
}

qd_status q4_0_quantize(const float *w, int64_t rows, int64_t cols, void *out,
                        void *stream) {
  if (!w || !out) return QD_EINVAL;
  if (rows < 1 || cols < 1) return QD_EINVAL;
  if (cols % 32 != 0) return QD_ESHAPE;
  const int64_t nb = rows * (cols / 32);
  if (rows > kMaxRows || nb > kMaxRows) return QD_EINVAL;
  if (!aligned(w, 16) || !aligned(out, 4)) return QD_EALIGN;
  if (overlap(out, q40_bytes(rows, cols), w, (size_t)rows * cols * 4))
    return QD_EINVAL;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = qd::launch_q4_0_quantize(w, nb, (uint8_t *)out,
                                          (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

qd_status qd_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
  if (!buf || !sink || bytes == 0) return QD_EINVAL;
  if (bytes % 1024 != 0) return QD_ESHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return QD_EALIGN;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = qd::launch_stream_read(buf, bytes, sink, (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

}  // extern "C"

extern "C" {

size_t qgemv_affine_i8_g64_step_workspace_bytes(const qd_affine_gemv_op *ops,
                                                int64_t n_ops, int64_t m) {
  if (!ops || n_ops < 1 || n_ops > kMaxStepOps) return 0;
  const std::vector<StepIn> v = step_in(ops, n_ops);
  return step_workspace_bytes(v.data(), n_ops, m, StepFormat{false});
}

qd_status qgemv_affine_i8_g64_step_plan(const qd_affine_gemv_op *ops,
                                        int64_t n_ops, int64_t m,
                                        void *workspace, size_t workspace_bytes,
                                        qd_step_plan *plan, void *stream) {
  if (!ops || n_ops < 1 || n_ops > kMaxStepOps) return QD_EINVAL;
  const std::vector<StepIn> v = step_in(ops, n_ops);
  return step_plan(v.data(), n_ops, m, StepFormat{false}, workspace, workspace_bytes, plan,
                   stream);
}

qd_status qgemv_affine_i8_g64_step_run(const qd_step_plan *plan, void *stream) {
  return step_run(plan, false, stream);
}

qd_status qgemv_affine_i8_g64_step_check(const qd_step_plan *plan,
                                         uint32_t *error_bits, void *stream) {
  return step_check(plan, false, error_bits, stream);
}

size_t qgemv_q4_0_step_workspace_bytes(const qd_q4_0_gemv_op *ops, int64_t n_ops, int64_t m) {
  if (!ops || n_ops < 1 || n_ops > kMaxStepOps) return 0;
  const std::vector<StepIn> v = step_in(ops, n_ops);
  return step_workspace_bytes(v.data(), n_ops, m, StepFormat{true});
}

qd_status qgemv_q4_0_step_plan(const qd_q4_0_gemv_op *ops, int64_t n_ops, int64_t m,
                               void *workspace, size_t workspace_bytes, qd_step_plan *plan,
                               void *stream) {
  if (!ops || n_ops < 1 || n_ops > kMaxStepOps) return QD_EINVAL;
  const std::vector<StepIn> v = step_in(ops, n_ops);
  return step_plan(v.data(), n_ops, m, StepFormat{true}, workspace, workspace_bytes, plan,
                   stream);
}

qd_status qgemv_q4_0_step_run(const qd_step_plan *plan, void *stream) {
  return step_run(plan, true, stream);
}

qd_status qgemv_q4_0_step_check(const qd_step_plan *plan, uint32_t *error_bits, void *stream) {
  return step_check(plan, true, error_bits, stream);
}

}  // extern "C"

static bool attention_shape_ok(int64_t heads, int64_t kv_heads, int64_t head_dim) {
  if (kv_heads < 1 || kv_heads > 65535 || heads < 1 || heads % kv_heads != 0) return false;
  const int64_t g = heads / kv_heads;
  return (g == 1 || g == 2 || g == 4 || g == 8) && (head_dim == 64 || head_dim == 128);
}

extern "C" {

int64_t attention_decode_workspace_bytes(int64_t heads, int64_t kv_heads, int64_t head_dim) {
  if (!attention_shape_ok(heads, kv_heads, head_dim)) return 0;
  return heads * qd::attention_max_chunks(kv_heads) * (head_dim + 2) * 4;
}

}  // extern "C"

// Host-side checks shared by attention_decode and attention_decode_noalloc
// (the workspace's own checks are the caller's); fills the kernels'
// arguments except the partials' buffer.  *need = the partials' bytes.
static qd_status attention_args(const void *q, const void *k_cache, const void *v_cache,
                                int64_t heads, int64_t kv_heads, int64_t head_dim,
                                int64_t length, int64_t kv_start, float scale, int32_t f16,
                                void *out, qd::AttentionArgs &a, int64_t &need) {
  if (!q || !k_cache || !v_cache || !out) return QD_EINVAL;
  if (f16 != 0 && f16 != 1) return QD_EINVAL;
  if (!attention_shape_ok(heads, kv_heads, head_dim)) return QD_ESHAPE;
  if (kv_start < 0 || kv_start >= length || length > (int64_t(1) << 30)) return QD_EINVAL;
  if (!std::isfinite(scale)) return QD_EINVAL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return QD_EALIGN;
  need = attention_decode_workspace_bytes(heads, kv_heads, head_dim);
  const size_t qb = (size_t)heads * head_dim * 2;
  const size_t cb = (size_t)length * kv_heads * head_dim * 2;
  const void *ins[3] = {q, k_cache, v_cache};
  const size_t insz[3] = {qb, cb, cb};
  for (int i = 0; i < 3; ++i)
    if (overlap(out, qb, ins[i], insz[i])) return QD_EINVAL;
  a = {};
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k_cache;
  a.v = (const uint16_t *)v_cache;
  a.out = (uint16_t *)out;
  a.heads = (int)heads;
  a.kv_heads = (int)kv_heads;
  a.head_dim = (int)head_dim;
  a.kv_start = (int)kv_start;
  a.length = (int)length;
  a.scale = scale;
  a.f16 = f16 == 1;
  a.pos_dev = nullptr;
  a.capacity = 0;
  a.qkr = nullptr;
  return QD_OK;
}

extern "C" {

qd_status attention_decode(const void *q, const void *k_cache, const void *v_cache,
                           int64_t heads, int64_t kv_heads, int64_t head_dim, int64_t length,
                           int64_t kv_start, float scale, int32_t f16, void *out,
                           void *workspace, size_t workspace_bytes, void *stream) {
  if (!workspace) return QD_EINVAL;
  qd::AttentionArgs a;
  int64_t need = 0;
  qd_status st = attention_args(q, k_cache, v_cache, heads, kv_heads, head_dim, length,
                                kv_start, scale, f16, out, a, need);
  if (st != QD_OK) return st;
  if (!aligned(workspace, 16)) return QD_EALIGN;
  if ((int64_t)workspace_bytes < need) return QD_EINVAL;
  const size_t qb = (size_t)heads * head_dim * 2;
  const size_t cb = (size_t)length * kv_heads * head_dim * 2;
  const void *ins[3] = {q, k_cache, v_cache};
  const size_t insz[3] = {qb, cb, cb};
  for (int i = 0; i < 3; ++i)
    if (overlap(workspace, (size_t)need, ins[i], insz[i])) return QD_EINVAL;
  if (overlap(out, qb, workspace, (size_t)need)) return QD_EINVAL;
  st = check_device();
  if (st != QD_OK) return st;
  a.part = (float *)workspace;
  hipError_t e = qd::launch_attention_decode(a, (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

qd_status attention_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                   int64_t heads, int64_t kv_heads, int64_t head_dim,
                                   int64_t length, int64_t kv_start, float scale, int32_t f16,
                                   void *out, void *stream) {
  qd::AttentionArgs a;
  int64_t need = 0;
  qd_status st = attention_args(q, k_cache, v_cache, heads, kv_heads, head_dim, length,
                                kv_start, scale, f16, out, a, need);
  if (st != QD_OK) return st;
  if ((uint64_t)need > qd::attention_noalloc_scratch_bytes()) return QD_ESCRATCH;
  st = check_device();
  if (st != QD_OK) return st;
  void *scratch = nullptr;
  hipError_t e = qd::attention_noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e);
  a.part = (float *)scratch;
  e = qd::launch_attention_decode(a, (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

}  // extern "C"

// ---- the decoder step around the GEMVs --------------------------------------

static bool finite_nonneg(float v) { return std::isfinite(v) && v >= 0.f; }

extern "C" {

qd_status rmsnorm_f16(void *x, const void *delta, const void *w, int64_t n, float eps,
                      void *out, void *stream) {
  if (!x || !w || !out || !finite_nonneg(eps)) return QD_EINVAL;
  if (n < 64 || n > 8192 || n % 64 != 0) return QD_ESHAPE;
  if (!aligned(x, 8) || !aligned(w, 8) || !aligned(out, 8) || (delta && !aligned(delta, 8)))
    return QD_EALIGN;
  const size_t nb = (size_t)n * 2;
  if (overlap(out, nb, x, nb) || overlap(out, nb, w, nb) || (delta && overlap(out, nb, delta, nb)))
    return QD_EINVAL;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = qd::launch_add_rmsnorm((const uint16_t *)x, (const uint16_t *)delta,
                                        (const uint16_t *)w, (int)n, eps, (uint16_t *)out,
                                        (uint16_t *)x, nullptr, (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

qd_status qk_norm_rope_f16(void *q, const void *k_src, const void *v_src, const void *q_norm,
                           const void *k_norm, int64_t heads, int64_t kv_heads, int64_t head_dim,
                           float eps, float theta, const int32_t *position, int64_t capacity,
                           void *k_cache, void *v_cache, uint32_t *error_word, void *stream) {
  if (!q || !k_src || !v_src || !q_norm || !k_norm || !position || !k_cache || !v_cache ||
      !error_word)
    return QD_EINVAL;
  if (heads < 1 || kv_heads < 1 || heads > 65535 || kv_heads > 65535 ||
      (head_dim != 64 && head_dim != 128))
    return QD_ESHAPE;
  if (capacity < 1 || capacity > (int64_t(1) << 30) || !finite_nonneg(eps) ||
      !std::isfinite(theta) || theta <= 0.f)
    return QD_EINVAL;
  const void *p2[] = {q, k_src, v_src, q_norm, k_norm, k_cache, v_cache};
  for (const void *p : p2)
    if (!aligned(p, 2)) return QD_EALIGN;
  if (!aligned(position, 4) || !aligned(error_word, 4)) return QD_EALIGN;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = qd::launch_qk_norm_rope(
      (uint16_t *)q, (const uint16_t *)k_src, (const uint16_t *)v_src, (const uint16_t *)q_norm,
      (const uint16_t *)k_norm, (int)heads, (int)kv_heads, (int)head_dim, eps, theta, position,
      (int)capacity, (uint16_t *)k_cache, (uint16_t *)v_cache, error_word, (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

qd_status silu_mul_f16(const void *gate, const void *up, void *out, int64_t n, void *stream) {
  if (!gate || !up || !out) return QD_EINVAL;
  if (n < 4 || n % 4 != 0 || n > (int64_t(1) << 30)) return QD_ESHAPE;
  if (!aligned(gate, 8) || !aligned(up, 8) || !aligned(out, 8)) return QD_EALIGN;
  const size_t nb = (size_t)n * 2;
  if (overlap(out, nb, up, nb) || (out != gate && overlap(out, nb, gate, nb))) return QD_EINVAL;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = qd::launch_silu_mul((const uint16_t *)gate, (const uint16_t *)up,
                                     (uint16_t *)out, (int)n, (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

}  // extern "C"

namespace {

// Byte offsets of the step workspace's parts (each 256-byte aligned).
struct StepLayout {
  size_t err, xalt, q, kbuf, vbuf, attn, delta, gate, up, part, opart, qrope, total;
};

// The o projection runs inside the attention's combine when the gate/up
// prologue can sum its per-K/V-head partial rows.
constexpr int64_t kStepMaxOParts = 8;
bool step_fused_o(const qd_qwen3_model &m) { return m.kv_heads <= kStepMaxOParts; }

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

bool qwen3_shape_ok(const qd_qwen3_model &m) {
  const int64_t qw = m.heads * m.head_dim;
  auto w64 = [](int64_t v) { return v >= 64 && v <= kMaxGemvCols && v % 64 == 0; };
  return w64(m.hidden) && w64(m.inter) && w64(qw) && attention_shape_ok(m.heads, m.kv_heads,
                                                                       m.head_dim) &&
         m.vocab >= 1 && m.vocab <= kMaxRows && m.n_layers >= 1 && m.capacity >= 1 &&
         m.capacity <= (int64_t(1) << 30);
}

StepLayout qwen3_layout(const qd_qwen3_model &m) {
  StepLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round256(bytes);
    return at;
  };
  const size_t qw = (size_t)m.heads * m.head_dim, kw = (size_t)m.kv_heads * m.head_dim;
  L.err = take(4);
  L.xalt = take(m.hidden * 2);
  L.q = take(qw * 2);
  L.kbuf = take(kw * 2);
  L.vbuf = take(kw * 2);
  L.attn = take(qw * 2);
  L.delta = take(m.hidden * 2);
  L.gate = take(m.inter * 2);
  L.up = take(m.inter * 2);
  L.part = take((size_t)attention_decode_workspace_bytes(m.heads, m.kv_heads, m.head_dim));
  L.opart = take(step_fused_o(m) ? (size_t)m.kv_heads * m.hidden * 4 : 0);
  L.qrope = take(qw * 2);
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

size_t qwen3_step_workspace_bytes(const qd_qwen3_model *model) {
  if (!model || !qwen3_shape_ok(*model)) return 0;
  return qwen3_layout(*model).total;
}

int64_t qwen3_step_workspace_offset(const qd_qwen3_model *model, int32_t buffer) {
  if (!model || !qwen3_shape_ok(*model)) return -1;
  const StepLayout L = qwen3_layout(*model);
  const bool fo = step_fused_o(*model);
  switch (buffer) {
    case QD_QWEN3_BUF_Q: return (int64_t)L.q;
    case QD_QWEN3_BUF_K: return (int64_t)L.kbuf;
    case QD_QWEN3_BUF_V: return (int64_t)L.vbuf;
    case QD_QWEN3_BUF_ATTN: return (int64_t)L.attn;
    case QD_QWEN3_BUF_OPART: return fo ? (int64_t)L.opart : -1;
    case QD_QWEN3_BUF_GATE: return (int64_t)L.gate;
    case QD_QWEN3_BUF_UP: return (int64_t)L.up;
    case QD_QWEN3_BUF_DELTA: return (int64_t)L.delta;
    case QD_QWEN3_BUF_XALT: return (int64_t)L.xalt;
    case QD_QWEN3_BUF_QROPE: return (int64_t)L.qrope;
    default: return -1;
  }
}

qd_status qwen3_step_run(const qd_qwen3_model *model, void *workspace, size_t workspace_bytes,
                         void *x, int32_t *position, void *logits, int32_t advance,
                         void *stream) {
  if (!model || !workspace || !x || !position || !model->layers || !model->final_norm ||
      !model->embed)
    return QD_EINVAL;
  if (advance != 0 && advance != 1) return QD_EINVAL;
  const qd_qwen3_model &m = *model;
  if (!qwen3_shape_ok(m)) return QD_ESHAPE;
  if (!finite_nonneg(m.eps) || !std::isfinite(m.theta) || m.theta <= 0.f) return QD_EINVAL;
  const StepLayout L = qwen3_layout(m);
  if (workspace_bytes < L.total) return QD_EINVAL;
  if (!aligned(workspace, 256) || !aligned(x, 16) || !aligned(position, 4) ||
      (logits && !aligned(logits, 2)) || !aligned(m.final_norm, 16) || !aligned(m.embed, 16))
    return QD_EALIGN;
  for (int64_t l = 0; l < m.n_layers; ++l) {
    const qd_qwen3_layer &ly = m.layers[l];
    const void *blobs[] = {ly.q, ly.k, ly.v, ly.o, ly.gate, ly.up, ly.down};
    const void *norms[] = {ly.in_norm, ly.q_norm, ly.k_norm, ly.post_norm};
    for (const void *p : blobs)
      if (!p) return QD_EINVAL;
    for (const void *p : norms)
      if (!p) return QD_EINVAL;
    if (!ly.k_cache || !ly.v_cache) return QD_EINVAL;
    for (const void *p : blobs)
      if (!aligned(p, 16)) return QD_EALIGN;
    for (const void *p : norms)
      if (!aligned(p, 16)) return QD_EALIGN;
    if (!aligned(ly.k_cache, 16) || !aligned(ly.v_cache, 16)) return QD_EALIGN;
  }
  const size_t hb = (size_t)m.hidden * 2;
  if (overlap(x, hb, workspace, L.total) ||
      (logits && (overlap(logits, (size_t)m.vocab * 2, workspace, L.total) ||
                  overlap(logits, (size_t)m.vocab * 2, x, hb))))
    return QD_EINVAL;
  // the caches (written by the step) clear of the workspace, x and logits
  const size_t cb = (size_t)m.capacity * m.kv_heads * m.head_dim * 2;
  for (int64_t l = 0; l < m.n_layers; ++l) {
    const void *caches[2] = {m.layers[l].k_cache, m.layers[l].v_cache};
    for (const void *c : caches)
      if (overlap(c, cb, workspace, L.total) || overlap(c, cb, x, hb) ||
          (logits && overlap(c, cb, logits, (size_t)m.vocab * 2)))
        return QD_EINVAL;
    if (overlap(caches[0], cb, caches[1], cb)) return QD_EINVAL;
  }
  qd_status st = check_device();
  if (st != QD_OK) return st;

  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  unsigned *err = (unsigned *)(ws + L.err);
  uint16_t *q = (uint16_t *)(ws + L.q);
  uint16_t *kbuf = (uint16_t *)(ws + L.kbuf), *vbuf = (uint16_t *)(ws + L.vbuf);
  uint16_t *attn = (uint16_t *)(ws + L.attn), *delta = (uint16_t *)(ws + L.delta);
  uint16_t *gate = (uint16_t *)(ws + L.gate), *up = (uint16_t *)(ws + L.up);
  float *opart = (float *)(ws + L.opart);
  // The residual row alternates between the caller's x and a scratch row:
  // a fused residual add reads one and writes the other, so no workgroup
  // reads a row that another is rewriting.  A step has 2 * n_layers adds,
  // so the final row lands in x again.
  uint16_t *res[2] = {(uint16_t *)x, (uint16_t *)(ws + L.xalt)};
  int cur = 0;
  const int hid = (int)m.hidden, d = (int)m.head_dim, H = (int)m.heads, KV = (int)m.kv_heads;
  const int qw = H * d, kw = KV * d, inter = (int)m.inter;
  const float scale = 1.0f / sqrtf((float)d);  // the page's f32 1/sqrt(head_dim)
  int *pos = (int *)position;
  hipError_t e = hipSuccess;
#define QD_TRY(call)                         \
  do {                                       \
    e = (call);                              \
    if (e != hipSuccess) return hip_fail(e); \
  } while (0)

  for (int64_t l = 0; l < m.n_layers; ++l) {
    const qd_qwen3_layer &ly = m.layers[l];
    // [residual add +] input RMSNorm, fused into the q/k/v GEMVs (one launch)
    qd::GemvPrologue pn = {};
    pn.kind = 1;
    pn.w = (const uint16_t *)ly.in_norm;
    pn.eps = m.eps;
    if (l > 0) {
      pn.delta = delta;
      pn.x_out = res[cur ^ 1];
    }
    qd::AffineGroup g = {};
    g.n = 3;
    g.w[0] = (const uint8_t *)ly.q;
    g.y[0] = q;
    g.rows[0] = qw;
    g.w[1] = (const uint8_t *)ly.k;
    g.y[1] = kbuf;
    g.rows[1] = kw;
    g.w[2] = (const uint8_t *)ly.v;
    g.y[2] = vbuf;
    g.rows[2] = kw;
    QD_TRY(qd::launch_affine_gemv_pro(g, hid, res[cur], pn, s));
    if (l > 0) cur ^= 1;
    // per-head norms + RoPE of q and the new K row, and the K/V append at
    // row p, fused into the attention's first kernel
    qd::AttentionQkRope qr = {};
    qr.q_out = (uint16_t *)(ws + L.qrope);
    qr.k_src = kbuf;
    qr.v_src = vbuf;
    qr.q_w = (const uint16_t *)ly.q_norm;
    qr.k_w = (const uint16_t *)ly.k_norm;
    qr.eps = m.eps;
    qr.theta = m.theta;
    qr.freq_ratio = std::pow((double)m.theta, -2.0 / (double)d);
    qr.err = err;
    qd::AttentionArgs a = {};
    a.q = q;
    a.k = (const uint16_t *)ly.k_cache;
    a.v = (const uint16_t *)ly.v_cache;
    a.out = attn;
    a.part = (float *)(ws + L.part);
    a.heads = H;
    a.kv_heads = KV;
    a.head_dim = d;
    a.kv_start = 0;
    a.length = 1;
    a.scale = scale;
    a.f16 = true;
    a.pos_dev = pos;
    a.capacity = (int)m.capacity;
    a.qkr = &qr;
    const bool fused_o = step_fused_o(m);
    if (fused_o) {
      // the o projection inside the combine: one fp32 partial row per K/V head
      a.wo = (const uint8_t *)ly.o;
      a.wo_rows = hid;
      a.wo_cols = qw;
      a.opart = opart;
    }
    QD_TRY(qd::launch_attention_decode(a, s));
    if (!fused_o) {
      qd::AffineGroup go = {};
      go.n = 1;
      go.w[0] = (const uint8_t *)ly.o;
      go.y[0] = delta;
      go.rows[0] = hid;
      QD_TRY(qd::launch_affine_gemv(go, qw, attn, 1, true, s));
    }
    // residual add (o = f16 of the partials' sum) + post-attention RMSNorm,
    // fused into the gate/up GEMVs
    qd::GemvPrologue pp = {};
    pp.kind = 1;
    if (fused_o) {
      pp.dparts = opart;
      pp.nparts = KV;
    } else {
      pp.delta = delta;
    }
    pp.w = (const uint16_t *)ly.post_norm;
    pp.x_out = res[cur ^ 1];
    pp.eps = m.eps;
    qd::AffineGroup gu = {};
    gu.n = 2;
    gu.w[0] = (const uint8_t *)ly.gate;
    gu.y[0] = gate;
    gu.rows[0] = inter;
    gu.w[1] = (const uint8_t *)ly.up;
    gu.y[1] = up;
    gu.rows[1] = inter;
    QD_TRY(qd::launch_affine_gemv_pro(gu, hid, res[cur], pp, s));
    cur ^= 1;
    // SiLU-mul, fused into the down GEMV
    qd::GemvPrologue ps = {};
    ps.kind = 2;
    ps.up = up;
    qd::AffineGroup gd = {};
    gd.n = 1;
    gd.w[0] = (const uint8_t *)ly.down;
    gd.y[0] = delta;
    gd.rows[0] = hid;
    QD_TRY(qd::launch_affine_gemv_pro(gd, inter, gate, ps, s));
  }
  // the last residual add; with logits, fused with the final norm into the
  // tied LM head
  if (logits) {
    qd::GemvPrologue pf = {};
    pf.kind = 1;
    pf.delta = delta;
    pf.w = (const uint16_t *)m.final_norm;
    pf.x_out = res[cur ^ 1];
    pf.advance = advance ? pos : nullptr;
    pf.eps = m.eps;
    qd::AffineGroup gl = {};
    gl.n = 1;
    gl.w[0] = (const uint8_t *)m.embed;
    gl.y[0] = (uint16_t *)logits;
    gl.rows[0] = (int)m.vocab;
    QD_TRY(qd::launch_affine_gemv_pro(gl, hid, res[cur], pf, s));
  } else {
    QD_TRY(qd::launch_add_rmsnorm(res[cur], delta, nullptr, hid, m.eps, nullptr, res[cur ^ 1],
                                  advance ? pos : nullptr, s));
  }
#undef QD_TRY
  return QD_OK;
}

qd_status qwen3_step_check(void *workspace, uint32_t *error_bits, void *stream) {
  if (!workspace || !error_bits) return QD_EINVAL;
  if (!aligned(workspace, 256)) return QD_EALIGN;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  uint32_t bits = 0;
  e = hipMemcpy(&bits, workspace, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e);
  *error_bits = bits;
  if (bits) {
    const uint32_t zero = 0;
    e = hipMemcpy(workspace, &zero, 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e);
    return QD_ESTEP;
  }
  return QD_OK;
}

}  // extern "C"
