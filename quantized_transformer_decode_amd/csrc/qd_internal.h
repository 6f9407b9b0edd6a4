// qd_internal.h -- launchers between the validated C entry points
// (qd_api.hip) and the kernels.  Arguments reaching these functions have
// already passed every host-side check; each launcher only enqueues work on
// `stream` and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qd {

// Compute units of the current device, cached per device (0 if unknown).
int device_cus();

// GEMVs of one launch that share their input x (and so `cols`): matrix k
// has rows[k] rows and owns the row tiles [tile0[k], tile0[k+1]) of the
// launch (tiles of the kernel's own height; the launcher fills tile0).
constexpr int kMaxGroup = 4;
struct AffineGroup {
  const uint8_t *w[kMaxGroup];
  uint16_t *y[kMaxGroup];
  int rows[kMaxGroup];
  int tile0[kMaxGroup + 1];
  int n;
  int grid;    // workgroups of the launch (set by the launcher)
  int ntiles;  // tile0[n] (set by the launcher)
  // ceil(2^32 / (cols / 8)): floor(i / (cols / 8)) = umulhi(i, xdiv) for the
  // 16-byte chunk indices of x (i * cols / 8 < 2^32); set by the launcher
  uint32_t xdiv;
};
// Q4_0 products of one launch, each with an optional f32 bias [rows] added
// to its outputs and, with gelu, gelu_tanh applied after it (q_linear).
struct Q40Group {
  const uint8_t *w[kMaxGroup];
  float *y[kMaxGroup];
  const float *bias[kMaxGroup];
  int rows[kMaxGroup];
  int tile0[kMaxGroup + 1];
  int n;
  int gelu;
  int grid;    // workgroups of the launch (set by the GEMV launcher)
  int ntiles;  // tile0[n] (set by the GEMV launcher)
};

// x and y BF16, or f16 with f16 = true (scales and biases BF16 in both).
hipError_t launch_affine_gemv(AffineGroup g, int cols, const uint16_t *x, int m, bool f16,
                              hipStream_t stream);

// An input transform fused into an f16 GEMV at m = 1 (the decoder step): the
// workgroups stage the transformed row in LDS instead of x itself.
//   kind 1, residual add + RMSNorm: a = x, or f16(x + delta) with delta;
//           the GEMV reads f16(a / sqrt(mean(a^2) + eps) * w) (w BF16);
//           workgroup 0 stores a to x_out (which must not be x) when delta
//           is given, and adds 1 to *advance when advance is given.
//   kind 2, SiLU-mul: the GEMV reads f16(silu(x) * up).
struct GemvPrologue {
  int kind;
  const uint16_t *delta, *w, *up;
  // kind 1 alternative to delta: f16(sum over nparts fp32 rows dparts[j][cols])
  const float *dparts;
  int nparts;
  uint16_t *x_out;
  int *advance;
  float eps;
};
hipError_t launch_affine_gemv_pro(AffineGroup g, int cols, const uint16_t *x,
                                  const GemvPrologue &pro, hipStream_t stream);

// Tied-embedding rows: token ids t[0..n) (already checked to be < rows).
constexpr int kMaxEmbedTokens = 16;
struct EmbedTokens {
  int t[kMaxEmbedTokens];
  int n;
};
hipError_t launch_affine_embed_rows(const uint8_t *w, int rows, int cols, const EmbedTokens &tk,
                                    uint16_t *out, bool f16, hipStream_t stream);

hipError_t launch_q4_0_gemv(Q40Group g, int cols, const float *x, int m,
                            hipStream_t stream);

hipError_t launch_q4_0_gemm(Q40Group g, int cols, const uint16_t *x, int m,
                            hipStream_t stream);

hipError_t launch_q4_0_quantize(const float *w, int64_t n_blocks, uint8_t *out,
                                hipStream_t stream);

// Decode attention over the K/V cache (attention.hip).  q, k, v and out are
// 16-bit (f16, else BF16); the cache rows are [rows][kv_heads][head_dim];
// part holds heads * nchunks * (head_dim + 2) floats of chunk partials.
// With pos_dev (device int32), the window is [0, *pos_dev + 1) of a cache of
// `capacity` rows (nothing is computed when the position is outside it) and
// kv_start / length are ignored.
// With qkr (device position and f16 only), q is the raw q/k/v GEMV output:
// the first kernel applies the per-head RMSNorm and NeoX RoPE of
// launch_qk_norm_rope to q (in registers) and to the new K row of k_src,
// which it appends, with the V row of v_src, at cache row *pos_dev; a
// position outside the cache sets bit 1 of *err.
struct AttentionQkRope {
  const uint16_t *k_src, *v_src, *q_w, *k_w;
  uint16_t *q_out;    // optional: the normed, rotated q rows (f16 [heads][head_dim])
  float eps, theta;
  double freq_ratio;  // theta^(-2 / head_dim) in fp64 (host)
  unsigned *err;
};
struct AttentionArgs {
  const uint16_t *q, *k, *v;
  uint16_t *out;
  float *part;
  int heads, kv_heads, head_dim, kv_start, length;
  float scale;
  bool f16;
  const int *pos_dev;
  int capacity;
  const AttentionQkRope *qkr;
  // Optional (f16, device position): the combine also applies the o
  // projection (affine-INT8 g64, wo_rows x wo_cols, wo_cols = heads *
  // head_dim) and writes opart[kv_heads][wo_rows] (fp32 partial rows, one
  // per K/V head); out, when not null, still receives the attention row.
  const uint8_t *wo;
  int wo_rows, wo_cols;
  float *opart;
};
// Rows per wave and chunks of the window [kv_start, length) (host only).
struct AttentionPlan {
  int rows_per_wave, nchunks;
};
AttentionPlan attention_plan(int64_t kv_heads, int64_t window, int head_dim);
// Upper bound of nchunks over every window (host only).
int64_t attention_max_chunks(int64_t kv_heads);
hipError_t launch_attention_decode(const AttentionArgs &a, hipStream_t stream);
// The library's static scratch for the chunk partials of the allocation-free
// attention entry point: its size, and its address on the current device
// (looked up once per device with hipGetSymbolAddress).
size_t attention_noalloc_scratch_bytes();
hipError_t attention_noalloc_scratch(void **ptr);

// Small ops of the decoder step (decoder_ops.hip), f16 buffers, BF16 norm
// weights.  add_rmsnorm: a = x, or f16(x + delta) stored to x_out (which may
// be x) when delta is given; then out = f16(rmsnorm(a) * w) (w optional),
// then *advance += 1 (optional); n % 4 == 0, n <= 8192.  qk_norm_rope: per-head RMSNorm + NeoX RoPE at
// *pos_dev of q (in place) and of k_src into K cache row *pos_dev, V row
// copied into the V cache; a position outside [0, capacity) sets bit 1 of
// *err and writes nothing.  silu_mul: out = f16(silu(gate) * up), n % 4 == 0.
hipError_t launch_add_rmsnorm(const uint16_t *x, const uint16_t *delta, const uint16_t *w, int n,
                              float eps, uint16_t *out, uint16_t *x_out, int *advance,
                              hipStream_t stream);
hipError_t launch_qk_norm_rope(uint16_t *q, const uint16_t *k_src, const uint16_t *v_src,
                               const uint16_t *q_w, const uint16_t *k_w, int heads, int kv_heads,
                               int d, float eps, float theta, const int *pos_dev, int capacity,
                               uint16_t *k_cache, uint16_t *v_cache, unsigned *err,
                               hipStream_t stream);
hipError_t launch_silu_mul(const uint16_t *gate, const uint16_t *up, uint16_t *out, int n,
                           hipStream_t stream);

// Practical HBM read ceiling (hbm_probe.hip): reads `bytes` (a multiple of
// 1024) once.
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink,
                              hipStream_t stream);

// Persistent decode-step kernel (decode_step.hip): one workgroup per CU;
// affine-INT8 g64 ops (BF16 in and out) or, with q4, Q4_0 ops (f32).
struct StepOp;
struct StepStage;
int step_compute_waves(bool q4, int m);  // compute waves per workgroup of the step kernel
bool step_compact(bool q4, int m);       // LDS holds only a workgroup's ops (else all)
hipError_t launch_step(bool q4, const StepOp *ops, const StepStage *stages, int n_stages, int m,
                       int xmax, int nwg, uint32_t *epoch_word, uint32_t *rel, uint32_t *ctr,
                       uint32_t *err, size_t lds_bytes, int group,
                       hipStream_t stream);  // group: items per register group, 4 or 3

}  // namespace qd
