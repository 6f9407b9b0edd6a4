/*
 * qdecode.h -- C ABI of libqdecode.so: dequantize-inside-the-matmul kernels
 * for token-by-token transformer decoders on AMD Instinct MI355X (gfx950).
 *
 * Two weight formats, both defined by the pages this library follows:
 *
 *  affine-INT8 g64  (turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs --
 *     PackedLinear::resident, load_packed_linear, embed_row_bytes)
 *     One resident buffer [codes | scales | biases] for a [rows, cols] matrix:
 *       codes   rows*cols bytes, code of (r, c) at byte r*cols + c (the
 *               checkpoint's U32 words [rows, cols/4] viewed little-endian);
 *       scales  BF16 [rows, cols/64] at byte offset rows*cols;
 *       biases  BF16 [rows, cols/64] at byte offset rows*cols + rows*(cols/64)*2;
 *     w[r, c] = q * scale[r, c/64] + bias[r, c/64].
 *
 *  ggml Q4_0  (fuel-transformers 0.19.1, src/models/lazy_quantized_whisper.rs
 *     -- module documentation, quantize_in_out_to_q4_0)
 *     A row-major stream of 18-byte blocks, block (n, b) for output row n and
 *     32-column block b at byte 18*(n*cols/32 + b): f16 delta d (little-endian)
 *     then 16 bytes whose low nibble is element j and high nibble element
 *     j+16; w = d * (q - 8).  The stream is zero-padded to a multiple of 4
 *     bytes (2 bytes when the block count is odd).
 *
 * Conventions for every entry point:
 *  - All matrix/vector pointers are DEVICE pointers owned by the caller.  The
 *    library never allocates, frees or retains them.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously; results are valid once the caller has
 *    synchronised the stream.  Device faults surface at that synchronisation.
 *  - Every argument is validated on the host before any HIP call, so a host
 *    without a GPU can exercise every error path.  On error nothing is
 *    enqueued and the output is untouched.
 *  - Matrices are row-major; activations x are [m, cols] and outputs y are
 *    [m, rows], both row-major and contiguous.  Outputs must not overlap
 *    inputs.  Inputs are never written.
 *  - Functions are reentrant and thread-safe; the only global state is a
 *    per-device cache of the architecture check.
 *  - None of the matmuls takes a bias input: the pages apply biases outside
 *    the matmul (q_linear) or refuse biased linears (load_packed_linear).
 */
#ifndef QDECODE_H
#define QDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QD_OK = 0,
  QD_EINVAL = 1,  /* null pointer, m or rows out of range, overlapping output */
  QD_ESHAPE = 2,  /* divisibility requirement on cols violated               */
  QD_EALIGN = 3,  /* pointer misaligned for the kernel's vector loads/stores  */
  QD_EDEVICE = 4, /* no current HIP device, or it is not gfx950               */
  QD_EHIP = 5,    /* the HIP runtime reported an error; see qd_last_hip_error */
  QD_ESTEP = 6,   /* a decode-step launch reported an error word (see _step_check) */
  QD_ESCRATCH = 7 /* the call needs more than the library's static scratch holds */
} qd_status;

/* Human-readable name of a status code (static storage; never NULL). */
const char *qd_status_string(int status);

/* The hipError_t of the most recent QD_EHIP on the calling thread (0 if none). */
int qd_last_hip_error(void);

/* Library version string, e.g. "qdecode 0.1.0 gfx950". */
const char *qd_version(void);

/* ---- layout helpers (pure host arithmetic; 0 on invalid arguments) ------ */

/* Byte size of the affine blob: rows*cols + 2 * rows*(cols/64)*2.
 * Requires rows >= 1, cols >= 64, cols % 64 == 0. */
size_t affine_i8_g64_bytes(int64_t rows, int64_t cols);
/* Byte offset of the BF16 scales inside the blob: rows*cols. */
size_t affine_i8_g64_scales_offset(int64_t rows, int64_t cols);
/* Byte offset of the BF16 biases inside the blob: rows*cols + rows*(cols/64)*2. */
size_t affine_i8_g64_biases_offset(int64_t rows, int64_t cols);
/* Byte size of a Q4_0 stream for [rows, cols]: rows*cols/32*18 rounded up
 * to a multiple of 4.  Requires rows >= 1, cols >= 32, cols % 32 == 0. */
size_t q4_0_bytes(int64_t rows, int64_t cols);

/* ---- affine-INT8 g64 ------------------------------------------------------ */

/* Packed-weight loader (turbospark-runtime 0.3.0, qwen3_asr_metal.rs --
 * load_packed_linear): validates the checkpoint triplet's shape and writes
 * the resident blob codes | scales | biases.
 *   codes_u32   device, U32 [rows, cols/4]   (rows*cols bytes)
 *   scales_bf16 device, BF16 [rows, cols/64]
 *   biases_bf16 device, BF16 [rows, cols/64]
 *   blob        device, affine_i8_g64_bytes(rows, cols) bytes, 16-byte aligned
 * Requires cols % 64 == 0 (QD_ESHAPE), rows >= 1, no overlap between blob and
 * the sources (QD_EINVAL).  Bit-exact byte copy. */
qd_status affine_i8_g64_pack(const void *codes_u32, const void *scales_bf16,
                             const void *biases_bf16, int64_t rows,
                             int64_t cols, void *blob, void *stream);

/* y = x W^T with W dequantised inside the kernel (w = q*scale + bias), fp32
 * accumulation, BF16 output rounded to nearest even
 * (turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::gemv,
 * embed_row_bytes for the dequantisation).
 *   w_packed  device, the affine blob for [rows, cols], 16-byte aligned
 *   x_bf16    device, BF16 [m, cols], 16-byte aligned
 *   y_bf16    device, BF16 [m, rows], 2-byte aligned (may sit at an offset
 *             inside a larger buffer, e.g. a K/V cache row)
 *   m         number of token rows, 1 <= m <= 16
 * Requires cols % 64 == 0 and 64 <= cols <= 8192 (QD_ESHAPE),
 * 1 <= rows < 2^31 (QD_EINVAL). */
qd_status qgemv_affine_i8_g64(const void *w_packed, int64_t rows, int64_t cols,
                              const void *x_bf16, void *y_bf16, int64_t m,
                              void *stream);

/* GEMVs that read the same input in one launch (the q, k, v projections, or
 * gate and up, of a decoder layer: turbospark-runtime 0.3.0,
 * qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step issues them on one input):
 * y_k = x W_k^T for k < n_items, each exactly as qgemv_affine_i8_g64 with
 * (items[k].w_packed, items[k].rows, cols, x_bf16, items[k].y_bf16, m).
 *   items     host array of n_items entries, 1 <= n_items <= 4; each
 *             w_packed: device affine blob [rows, cols], 16-byte aligned;
 *             y_bf16: device BF16 [m, rows], 2-byte aligned; rows >= 1
 *   x_bf16    device, BF16 [m, cols], 16-byte aligned, shared by all items
 * Requirements and errors as qgemv_affine_i8_g64; in addition no output may
 * overlap another item's output or weights (QD_EINVAL). */
typedef struct {
  const void *w_packed;
  void *y_bf16;
  int64_t rows;
} qd_affine_gemv_item;

qd_status qgemv_affine_i8_g64_group(const qd_affine_gemv_item *items, int64_t n_items,
                                    int64_t cols, const void *x_bf16, int64_t m,
                                    void *stream);

/* The same GEMV with f16 activations, the dtype of the page's Metal GEMV
 * (turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::gemv
 * reads and writes f16 buffers): x f16 [m, cols], y f16 [m, rows] rounded to
 * nearest even from the fp32 accumulator (f16 subnormals kept, overflow to
 * infinity); scales and biases stay BF16 in the blob.  Arguments, alignment
 * and status codes as qgemv_affine_i8_g64. */
qd_status qgemv_affine_i8_g64_f16(const void *w_packed, int64_t rows, int64_t cols,
                                  const void *x_f16, void *y_f16, int64_t m, void *stream);

/* Tied-embedding rows on the device (turbospark-runtime 0.3.0,
 * qwen3_asr_metal.rs -- embed_row_bytes): out[i, c] = q*scale + bias of row
 * token_ids[i] of the packed matrix, evaluated in f32 (the product is exact,
 * the sum rounds once) and rounded to f16 (out_f16 = 1, the page's store) or
 * BF16 (out_f16 = 0), nearest even -- bit-exact.
 *   w_packed   device, the affine blob for [rows, cols], 16-byte aligned
 *   token_ids  host, n ids, each 0 <= id < rows (QD_EINVAL otherwise)
 *   n          1 <= n <= 16
 *   out        device, 16-bit [n, cols], 8-byte aligned; must not overlap
 *              the blob
 * Requires cols % 64 == 0 and cols <= 8192 (QD_ESHAPE). */
qd_status affine_i8_g64_embed_rows(const void *w_packed, int64_t rows, int64_t cols,
                                   const int64_t *token_ids, int64_t n, void *out,
                                   int32_t out_f16, void *stream);

/* ---- one decode step of affine GEMVs in a single launch ------------------ */

/* One GEMV of a decode step: y[m, rows] = x[m, cols] W^T (same operation,
 * layouts and rounding as qgemv_affine_i8_g64).  `stage` orders the GEMVs:
 * stages are numbered 0, 1, 2, ... in op-array order; GEMVs of one stage may
 * run concurrently (e.g. q, k, v, or gate and up, which read the same
 * input), and no GEMV of stage s+1 reads its input before every GEMV of
 * stage s has finished -- the decoder order of turbospark-runtime 0.3.0,
 * qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step. */
typedef struct {
  const void *w_packed; /* device, affine blob [rows, cols], 16-byte aligned */
  const void *x_bf16;   /* device, BF16 [m, cols], 16-byte aligned         */
  void *y_bf16;         /* device, BF16 [m, rows], 2-byte aligned          */
  int64_t rows, cols;   /* rows >= 1; cols % 64 == 0, 64 <= cols <= 8192   */
  int64_t stage;
} qd_affine_gemv_op;

/* Host-side handle filled by _step_plan (caller-owned plain data).  When
 * the last stage is a single GEMV of at least 2^27 weights (an LM head),
 * `tail` is 1 and that GEMV is kept here: _step_run streams it with the
 * single-GEMV kernel after the persistent kernel (which then runs the other
 * stages), because one matrix streamed by the persistent kernel's
 * whole-chip stage reaches about half the bandwidth of the streaming
 * kernel. */
typedef struct {
  void *workspace;
  int32_t nwg;        /* workgroups = CUs of the planning device */
  int32_t lds_bytes;
  int32_t n_ops, n_stages, m;
  uint32_t magic;
  int32_t tail;       /* 1: the last stage runs as a separate streaming GEMV */
  const void *tail_w, *tail_x;
  void *tail_y;
  int64_t tail_rows, tail_cols;
  int32_t format;     /* 0: affine-INT8 g64 plan, 1: Q4_0 plan (qgemv_q4_0_step_*) */
  int32_t group;      /* weight chunks per register group of a compute wave:
                         4 when the plan's stages give each wave more than
                         three on average (single-row affine plans), else 3 */
} qd_step_plan;

/* Workspace bytes needed by _step_plan for these ops (0 if invalid). */
size_t qgemv_affine_i8_g64_step_workspace_bytes(const qd_affine_gemv_op *ops,
                                                int64_t n_ops, int64_t m);

/* Validates the ops (host array), writes the step tables into `workspace`
 * (device memory owned by the caller, 256-byte aligned, at least
 * _step_workspace_bytes) and fills *plan.  Synchronises `stream` before
 * returning.  m is the number of token rows, 1 <= m <= 4 (QD_EINVAL
 * otherwise; every op's x is [m, cols] and y [m, rows]).  Requirements
 * beyond those of each op: ops[0].stage == 0 and each op's stage equals its
 * predecessor's or one more; ops of one stage share cols; the staged input
 * of a stage fits a workgroup's LDS -- at m = 1 sum(ceil(cols/1024)*1024)
 * over the stage's ops <= 16384, at m > 1 the same sum times m over the ops
 * any one workgroup has rows in (the stage's rows split evenly over the
 * device's compute units) -- and sum(m*cols) <= 128 * (compute units of the
 * device) (QD_ESHAPE; the last bound only binds on parts with fewer than
 * 128 CUs); no op's output overlaps any op's weights or input, or the
 * workspace (QD_EINVAL / QD_ESHAPE / QD_EALIGN as for the single GEMV).
 * The workspace, weights and inputs must stay valid while runs are in
 * flight. */
qd_status qgemv_affine_i8_g64_step_plan(const qd_affine_gemv_op *ops,
                                        int64_t n_ops, int64_t m,
                                        void *workspace, size_t workspace_bytes,
                                        qd_step_plan *plan, void *stream);

/* Enqueues the whole step as ONE persistent kernel (one workgroup per CU,
 * one kernel per token-row count;
 * every workgroup must be able to be resident, so do not run it concurrently
 * with kernels that occupy whole CUs indefinitely) and, with plan->tail,
 * the last stage's GEMV as a second launch on the same stream (it starts
 * after the persistent kernel has finished every other stage).  Launches
 * nothing else, allocates nothing, and may be captured in a HIP graph.  Runs
 * planned on the same workspace must not overlap in time.  After a run that
 * reported an error (qgemv_affine_i8_g64_step_check), plan again before the
 * next run: the workspace's arrival counts no longer match. */
qd_status qgemv_affine_i8_g64_step_run(const qd_step_plan *plan, void *stream);

/* Synchronises `stream`, reads the workspace's error word into *error_bits
 * (0 = every wait completed) and returns QD_ESTEP if it is non-zero.  Bits:
 * 1 input poll timed out, 2/4 intra-workgroup wait timed out, 8 grid size did
 * not match the plan. */
qd_status qgemv_affine_i8_g64_step_check(const qd_step_plan *plan,
                                         uint32_t *error_bits, void *stream);

/* The same single-launch step for Q4_0 GEMVs (the projections of a Whisper
 * decoder layer in decoder order: fuel-transformers 0.19.1,
 * lazy_quantized_whisper.rs -- decoder_layer applies q, k, v, then o, then
 * fc1, then fc2): y[m, rows] = x[m, cols] W^T with the operation, layouts and
 * f32 arithmetic of qgemv_q4_0 (no bias or GELU: q_linear's epilogue stays
 * with qlinear_q4_0_gemv).  Stage rules as qd_affine_gemv_op. */
typedef struct {
  const void *w_q4_0; /* device, Q4_0 stream [rows, cols], 16-byte aligned   */
  const float *x;     /* device, f32 [m, cols], 16-byte aligned             */
  float *y;           /* device, f32 [m, rows], 4-byte aligned              */
  int64_t rows, cols; /* rows >= 1; cols % 256 == 0, 256 <= cols <= 8192    */
  int64_t stage;
} qd_q4_0_gemv_op;

/* Workspace bytes needed by qgemv_q4_0_step_plan for these ops (0 if
 * invalid). */
size_t qgemv_q4_0_step_workspace_bytes(const qd_q4_0_gemv_op *ops, int64_t n_ops, int64_t m);

/* As qgemv_affine_i8_g64_step_plan, for Q4_0 ops: m == 1; ops of one stage
 * share cols; per stage sum(m*ceil(cols/2048)*2048) <= 16384 and
 * sum(m*cols) <= 64 * (compute units of the device) (QD_ESHAPE); no output
 * may overlap any op's weights, input or output, or the workspace
 * (QD_EINVAL).  Sets plan->format = 1 and plan->tail = 0 (every stage runs in
 * the persistent kernel). */
qd_status qgemv_q4_0_step_plan(const qd_q4_0_gemv_op *ops, int64_t n_ops, int64_t m,
                               void *workspace, size_t workspace_bytes, qd_step_plan *plan,
                               void *stream);

/* Enqueues a Q4_0 plan as ONE persistent kernel, with the guarantees and
 * limits of qgemv_affine_i8_g64_step_run.  QD_EINVAL for a plan of the other
 * format (and _step_run of the affine format rejects a Q4_0 plan). */
qd_status qgemv_q4_0_step_run(const qd_step_plan *plan, void *stream);

/* qgemv_affine_i8_g64_step_check for a Q4_0 plan (same error bits). */
qd_status qgemv_q4_0_step_check(const qd_step_plan *plan, uint32_t *error_bits, void *stream);

/* ---- ggml Q4_0 ------------------------------------------------------------ */

/* y = x W^T over a Q4_0 stream, f32 activations and f32 output
 * (fuel-transformers 0.19.1, lazy_quantized_whisper.rs -- q_linear /
 * WeightStorage::apply_linear; the bias is applied outside).
 *   w_q4_0  device, the Q4_0 stream for [rows = out_features, cols =
 *           in_features], 16-byte aligned
 *   x       device, f32 [m, cols], 16-byte aligned
 *   y       device, f32 [m, rows], 4-byte aligned
 *   m       1 <= m <= 16
 * Requires cols % 256 == 0 and 256 <= cols <= 8192 (QD_ESHAPE): every row
 * then starts on a 16-byte boundary (8 blocks = 144 bytes). */
qd_status qgemv_q4_0(const void *w_q4_0, int64_t rows, int64_t cols,
                     const float *x, float *y, int64_t m, void *stream);

/* Q4_0 GEMVs that read the same input in one launch (the self-attention q,
 * k, v projections of a Whisper decoder layer: fuel-transformers 0.19.1,
 * lazy_quantized_whisper.rs -- decoder_layer applies them to one input):
 * y_k = x W_k^T for k < n_items, each exactly as qgemv_q4_0 with
 * (items[k].w_q4_0, items[k].rows, cols, x, items[k].y, m).
 *   items   host array of n_items entries, 1 <= n_items <= 4; each w_q4_0:
 *           device Q4_0 stream [rows, cols], 16-byte aligned; y: device f32
 *           [m, rows], 4-byte aligned; rows >= 1
 *   x       device, f32 [m, cols], 16-byte aligned, shared by all items
 * Requirements and errors as qgemv_q4_0; in addition no output may overlap
 * another item's output or weights (QD_EINVAL). */
typedef struct {
  const void *w_q4_0;
  float *y;
  int64_t rows;
} qd_q4_0_gemv_item;

qd_status qgemv_q4_0_group(const qd_q4_0_gemv_item *items, int64_t n_items, int64_t cols,
                           const float *x, int64_t m, void *stream);

/* Prefill GEMM y = x W^T over a Q4_0 stream on the matrix cores: BF16
 * activations, exact integer codes (q - 8) as BF16 MFMA operands, the f16
 * delta applied per block in fp32, f32 output
 * (fuel-transformers 0.19.1, lazy_quantized_whisper.rs -- forward_encoder /
 * encoder_layer, which run every projection over all encoder frames).
 *   w_q4_0  device, Q4_0 stream for [rows, cols], 16-byte aligned
 *   x_bf16  device, BF16 [m, cols], 16-byte aligned
 *   y       device, f32 [m, rows], 16-byte aligned
 *   m       any 1 <= m <= 2^22 (the tail tile is masked)
 * Requires cols % 256 == 0, 256 <= cols <= 65536 (QD_ESHAPE). */
qd_status qgemm_q4_0_prefill(const void *w_q4_0, int64_t rows, int64_t cols,
                             const void *x_bf16, float *y, int64_t m,
                             void *stream);

/* q_linear: the Q4_0 product, then an optional f32 bias [rows] broadcast
 * over the token rows, then optionally gelu_tanh, the tanh form of GELU
 * 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
 * (fuel-transformers 0.19.1, lazy_quantized_whisper.rs -- q_linear, and
 * encoder_layer / decoder_layer, which apply gelu_tanh after fc1).  Up to
 * four products that read the same x share one launch (a layer's q, k, v:
 * 3 x 1280 output columns).
 *   w_q4_0  device, Q4_0 stream [rows, cols], 16-byte aligned
 *   bias    device, f32 [rows], 4-byte aligned, or NULL (k has none)
 *   y       device, f32 [m, rows] (GEMV: 4-byte, GEMM: 16-byte aligned)
 *   rows    1 <= rows < 2^31 */
typedef struct qd_q4_0_linear_item {
  const void *w_q4_0;
  const float *bias;
  float *y;
  int64_t rows;
} qd_q4_0_linear_item;

/* GEMV form: x f32 [m, cols], 1 <= m <= 16, cols % 256 == 0, cols <= 8192;
 * gelu 0 or 1.  No output may overlap x, any weights, any bias or another
 * output (QD_EINVAL).  Status codes as qgemv_q4_0_group. */
qd_status qlinear_q4_0_gemv(const qd_q4_0_linear_item *items, int64_t n_items, int64_t cols,
                            const float *x, int64_t m, int32_t gelu, void *stream);

/* GEMM (prefill) form on the matrix cores: x BF16 [m, cols], any m >= 1,
 * cols % 256 == 0, cols <= 65536; otherwise as qlinear_q4_0_gemv. */
qd_status qlinear_q4_0_gemm(const qd_q4_0_linear_item *items, int64_t n_items, int64_t cols,
                            const void *x_bf16, int64_t m, int32_t gelu, void *stream);

/* f32 -> Q4_0 bake (fuel-transformers 0.19.1, lazy_quantized_whisper.rs --
 * quantize_in_out_to_q4_0 with ggml's BlockQ4_0::from_float): per block of
 * 32, d = (element of largest magnitude, first index on ties) / -8 in f32,
 * id = 1/d correctly rounded (0 if d == 0), nibble = min(15, trunc(x*id +
 * 8.5)) with the product and the sum rounded separately (no FMA), d stored
 * as f16 round-to-nearest-even; blocks row-major; 2 zero bytes appended when
 * the block count is odd.  Bit-exact.  Non-finite inputs, or a block whose
 * |max|/8 overflows f16, are outside the contract (not checked).
 *   w    device, f32 [rows = out_features, cols = in_features], 16-byte
 *        aligned (callers holding [in, out] weights transpose first)
 *   out  device, q4_0_bytes(rows, cols) bytes, 4-byte aligned
 * Requires cols % 32 == 0 (QD_ESHAPE), rows >= 1 and rows*cols/32 < 2^31
 * (QD_EINVAL). */
qd_status q4_0_quantize(const float *w, int64_t rows, int64_t cols, void *out,
                        void *stream);

/* ---- decode attention over the K/V cache ---------------------------------- */

/* Bytes of the attention_decode workspace for this head shape (0 if the
 * shape is not supported): a bound over every window length. */
int64_t attention_decode_workspace_bytes(int64_t heads, int64_t kv_heads, int64_t head_dim);

/* Grouped-query decode attention for one token (turbospark-runtime 0.3.0,
 * qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step, encode_attention_decode
 * with its split-softmax scratch): for every query head h, with K/V head
 * j = h / (heads / kv_heads),
 *   out[h] = sum_t softmax_t(scale * q[h] . k[t, j]) v[t, j],
 *   t in [kv_start, length)
 * (the page attends the causal prefix: kv_start 0, length position + 1,
 * scale 1/sqrt(head_dim)).  Scores, exponentials and sums in fp32, the
 * output rounded once (nearest even) to the 16-bit type.  Workgroups take
 * chunks of the window (split softmax) and a second launch merges the
 * chunks of each head; a window of up to 128 rows is one chunk and takes
 * one launch.
 *   q          device, [heads, head_dim] 16-bit, 16-byte aligned
 *   k_cache,   device, [>= length rows, kv_heads, head_dim] 16-bit (the
 *   v_cache    cache row of position t holds every K/V head), 16-byte aligned
 *   heads, kv_heads  heads % kv_heads == 0 with heads / kv_heads in
 *              {1, 2, 4, 8} and 1 <= kv_heads <= 65535 (QD_ESHAPE)
 *   head_dim   64 or 128 (QD_ESHAPE)
 *   length, kv_start  0 <= kv_start < length <= 2^30 (QD_EINVAL)
 *   scale      finite (QD_EINVAL)
 *   f16        1: q, caches and out are f16 (the page's type); 0: BF16
 *   out        device, [heads, head_dim] 16-bit, 16-byte aligned
 *   workspace  device, f32 scratch for the chunk partials, 16-byte
 *              aligned, at least attention_decode_workspace_bytes(heads,
 *              kv_heads, head_dim) bytes (QD_EINVAL otherwise; the size does
 *              not depend on the window, so one workspace serves every call
 *              of a head shape); its contents on entry do not matter and are
 *              unspecified afterwards
 * out may overlap neither the inputs nor the workspace, nor the workspace
 * the inputs (QD_EINVAL).  Asynchronous on `stream`; calls sharing one
 * workspace must be ordered on one stream. */
qd_status attention_decode(const void *q, const void *k_cache, const void *v_cache,
                           int64_t heads, int64_t kv_heads, int64_t head_dim, int64_t length,
                           int64_t kv_start, float scale, int32_t f16, void *out,
                           void *workspace, size_t workspace_bytes, void *stream);

/* attention_decode for callers that cannot allocate (code under HIP graph
 * capture, serving loops that forbid allocation, harnesses without an
 * allocator): the same operation, arguments and errors as attention_decode
 * without the workspace.  The chunk partials go to a scratch buffer inside
 * the library -- a static device array of ATTENTION_NOALLOC_SCRATCH_BYTES
 * (4 MiB) that every device the library runs on holds until the process
 * ends.  A head shape whose attention_decode_workspace_bytes exceeds it is
 * rejected with QD_ESCRATCH before any HIP call.  This call allocates
 * nothing (no hipMalloc, no library routine that allocates); the first call
 * on a device looks the array's address up once.  All calls on one device
 * share the array and nothing in it needs to start at zero, but calls that
 * may overlap in time on one device (different streams, or different host
 * threads without ordering) race on it: order them on one stream. */
#define ATTENTION_NOALLOC_SCRATCH_BYTES (4u << 20)
qd_status attention_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                   int64_t heads, int64_t kv_heads, int64_t head_dim,
                                   int64_t length, int64_t kv_start, float scale, int32_t f16,
                                   void *out, void *stream);

/* ---- the decoder step around the GEMVs ------------------------------------ */

/* turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step
 * and the ops it encodes.  Every activation buffer is f16 (the page's
 * buffers), norm weights are BF16; each op computes in fp32 and rounds its
 * result to f16 once, where the page stores it. */

/* encode_residual_add + encode_rms_norm_bf16w: when delta is not NULL,
 * x <- f16(x + delta) (written back; the page's residual add); then
 * out = f16(x / sqrt(mean(x^2) + eps) * w).
 *   x      device, f16 [n], 8-byte aligned (in/out)
 *   delta  device, f16 [n], 8-byte aligned, or NULL
 *   w      device, BF16 [n], 8-byte aligned
 *   out    device, f16 [n], 8-byte aligned; may not overlap x, delta or w
 * Requires n % 64 == 0 and 64 <= n <= 8192 (QD_ESHAPE), eps finite and
 * >= 0 (QD_EINVAL).  One workgroup; asynchronous on `stream`. */
qd_status rmsnorm_f16(void *x, const void *delta, const void *w, int64_t n, float eps,
                      void *out, void *stream);

/* encode_rms_norm_bf16w_perhead + encode_rope_neox_subdim (rotary width =
 * head_dim) on q and on the new K row, which then lands in the cache, and
 * the V row copied into the cache: with p = *position (device int32),
 *   q[h]           <- f16(rope(f16(rmsnorm(q[h]) * q_norm), p))   (in place)
 *   k_cache[p, j]  <- f16(rope(f16(rmsnorm(k_src[j]) * k_norm), p))
 *   v_cache[p, j]  <- v_src[j]
 * where rope turns the pair (i, i + d/2) by p * theta^(-2i/d) (angle and its
 * sine and cosine in fp64, the rotation in fp32).
 *   q, k_src, v_src  device, f16 [heads * d] / [kv_heads * d] / [kv_heads * d]
 *   q_norm, k_norm   device, BF16 [head_dim]
 *   position         device, one int32; a value outside [0, capacity) writes
 *                    nothing and sets bit 1 of *error_word
 *   k_cache, v_cache device, f16 [capacity, kv_heads, head_dim]
 *   error_word       device, one uint32 (bits are only ever set)
 * Requires head_dim 64 or 128 and heads, kv_heads >= 1 (QD_ESHAPE),
 * 1 <= capacity <= 2^30, eps >= 0 and theta > 0 finite (QD_EINVAL), every
 * pointer non-NULL (QD_EINVAL) and 2-byte aligned (QD_EALIGN). */
qd_status qk_norm_rope_f16(void *q, const void *k_src, const void *v_src, const void *q_norm,
                           const void *k_norm, int64_t heads, int64_t kv_heads, int64_t head_dim,
                           float eps, float theta, const int32_t *position, int64_t capacity,
                           void *k_cache, void *v_cache, uint32_t *error_word, void *stream);

/* encode_silu_mul: out = f16(silu(gate) * up), silu(g) = g / (1 + e^-g).
 * gate, up, out: device f16 [n], 8-byte aligned; out may be gate (the page
 * writes gate in place) but may not overlap up otherwise.  n % 4 == 0,
 * n >= 4 (QD_ESHAPE). */
qd_status silu_mul_f16(const void *gate, const void *up, void *out, int64_t n, void *stream);

/* One decoder layer's weights (device pointers). */
typedef struct {
  const void *q, *k, *v, *o, *gate, *up, *down; /* affine blobs, 16-byte aligned */
  const void *in_norm, *q_norm, *k_norm, *post_norm; /* BF16 vectors, 16-byte aligned */
  void *k_cache, *v_cache; /* f16 [capacity, kv_heads, head_dim], 16-byte aligned */
} qd_qwen3_layer;

/* A Qwen3 text decoder in the page's storage forms (host struct; `layers`
 * is a host array of n_layers entries). */
typedef struct {
  int64_t hidden, heads, kv_heads, head_dim, inter, vocab, n_layers, capacity;
  float eps, theta;            /* rms_norm_eps, rope_theta */
  const qd_qwen3_layer *layers;
  const void *final_norm;      /* BF16 [hidden], 16-byte aligned */
  const void *embed;           /* affine blob [vocab, hidden]: the tied LM head */
} qd_qwen3_model;

/* Bytes of the step workspace for this model (0 if the model is not
 * supported): one error word, the f16 scratch rows, the attention partials,
 * with at most 8 K/V heads kv_heads fp32 rows of hidden entries (the o
 * projection's partial sums, one row per K/V head), and the rotated q row. */
size_t qwen3_step_workspace_bytes(const qd_qwen3_model *model);

/* The step's scratch rows inside the workspace (the page's `Work` buffers
 * that the fused kernels still store).  After a step they hold the last
 * layer's values:
 *   QD_QWEN3_BUF_Q      f16 [heads*head_dim]  q GEMV output, before its norm and RoPE
 *   QD_QWEN3_BUF_K      f16 [kv_heads*head_dim]  k GEMV output, before its norm and RoPE
 *   QD_QWEN3_BUF_V      f16 [kv_heads*head_dim]  v GEMV output
 *   QD_QWEN3_BUF_QROPE  f16 [heads*head_dim]  q after its per-head norm and RoPE
 *                       (the page's q buffer after encode_rope_neox_subdim)
 *   QD_QWEN3_BUF_ATTN   f16 [heads*head_dim]  attention output
 *   QD_QWEN3_BUF_OPART  fp32 [kv_heads][hidden]  the o projection's partial rows,
 *                       one per K/V head (kv_heads <= 8)
 *   QD_QWEN3_BUF_GATE   f16 [inter]  gate GEMV output (before SiLU)
 *   QD_QWEN3_BUF_UP     f16 [inter]  up GEMV output
 *   QD_QWEN3_BUF_DELTA  f16 [hidden]  down GEMV output (the o output when
 *                       kv_heads > 8, until the down GEMV overwrites it)
 *   QD_QWEN3_BUF_XALT   f16 [hidden]  the residual row after the attention block
 * Returns the byte offset of that row in the workspace, or -1 when the
 * model is not supported or the buffer is not used for this model.
 * Host-only arithmetic (no device call). */
enum {
  QD_QWEN3_BUF_Q = 0, QD_QWEN3_BUF_K = 1, QD_QWEN3_BUF_V = 2, QD_QWEN3_BUF_ATTN = 3,
  QD_QWEN3_BUF_OPART = 4, QD_QWEN3_BUF_GATE = 5, QD_QWEN3_BUF_UP = 6, QD_QWEN3_BUF_DELTA = 7,
  QD_QWEN3_BUF_XALT = 8, QD_QWEN3_BUF_QROPE = 9
};
int64_t qwen3_step_workspace_offset(const qd_qwen3_model *model, int32_t buffer);

/* Qwen3AsrMetalEngine::step for one row: x (device, f16 [hidden], 16-byte
 * aligned) goes through every layer at p = *position (device int32) --
 * rmsnorm, the q/k/v GEMVs (one launch), per-head q/k norms and RoPE with
 * the K/V rows appended at cache row p, decode attention over rows [0, p],
 * the o GEMV, residual add, rmsnorm, the gate/up GEMVs (one launch),
 * silu*mul, the down GEMV, residual add -- leaving the new residual row in
 * x.  With at most 8 K/V heads the o GEMV runs inside the attention's
 * combine as one fp32 partial per K/V head over that head's input columns,
 * summed in head order and rounded to f16 by the next launch; the o output
 * is then that sum instead of one fp32 sum over all columns.  When logits (device, f16 [vocab], 2-byte aligned) is not NULL, the
 * final norm and the tied LM-head GEMV write the next-token logits.  With
 * advance = 1, *position is incremented at the end of the step.  The
 * kernels read p from device memory, allocate nothing and launch no memset,
 * so the caller may capture one call in a HIP graph and replay it token
 * after token (with advance = 1).  A position outside [0, capacity) makes
 * the step write nothing to the caches and sets bit 1 of the workspace's
 * error word (qwen3_step_check).
 *   workspace  device, 256-byte aligned, >= qwen3_step_workspace_bytes;
 *              zero-filled before its first use (the error word)
 * Model requirements (QD_ESHAPE): hidden, inter and heads * head_dim
 * multiples of 64 and <= 8192; head_dim 64 or 128; heads / kv_heads in
 * {1, 2, 4, 8}; vocab, n_layers >= 1; 1 <= capacity <= 2^30.  Null or
 * misaligned pointers: QD_EINVAL / QD_EALIGN; x, logits, the workspace and
 * a layer's K and V caches must not overlap one another (QD_EINVAL).  Calls
 * sharing a workspace must be ordered on one stream. */
qd_status qwen3_step_run(const qd_qwen3_model *model, void *workspace, size_t workspace_bytes,
                         void *x, int32_t *position, void *logits, int32_t advance,
                         void *stream);

/* Synchronises `stream`, returns the workspace's error word in *error_bits
 * and clears it; QD_ESTEP if it was non-zero (bit 1: a position outside
 * [0, capacity)). */
qd_status qwen3_step_check(void *workspace, uint32_t *error_bits, void *stream);

/* ---- measurement aid (not a step of the decode path) ---------------------- */

/* Reads `bytes` bytes of device memory at `buf` once, with the access pattern
 * of the GEMV weight streams (every wave reads contiguous 1 KiB chunks with
 * 16-byte non-temporal loads, many chunks in flight), so that bytes / time
 * is a practical HBM read ceiling to set the GEMV rooflines against (the
 * 8 TB/s figure is the interface's peak).  buf: device, 16-byte aligned;
 * bytes: a positive multiple of 1024; sink: device, one uint32 that keeps
 * the loads live (its value afterwards is unspecified).  QD_EINVAL (null
 * pointer, bytes 0), QD_ESHAPE (bytes % 1024), QD_EALIGN; asynchronous on
 * `stream`. */
qd_status qd_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QDECODE_H */
