/*
 * qd_oracle.c -- plain, slow, obviously correct CPU oracle for the
 * dequantize-inside-the-matmul decode path (affine-INT8 g64 and ggml Q4_0).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library) never links, loads or calls it, and this file includes
 * nothing from the product sources.
 *
 * Arithmetic: every dot product is formed in IEEE double with a sequential
 * sum over the reduction index; every stored half / bfloat16 value is decoded
 * from its bit layout here.  The Q4_0 encoder is an encoding, not an
 * approximation, so it is written step by step in IEEE single precision and
 * must be compiled with -ffp-contract=off (no fused multiply-add).
 *
 * Sources (page title -- section):
 *   [P3] turbospark-runtime 0.3.0, src/qwen3_asr_metal.rs
 *        -- PackedLinear::resident (offsets of codes / scales / biases),
 *        -- load_packed_linear (dtype, shape and byte-count contract; blob
 *           order weight | scales | biases),
 *        -- embed_row_bytes (the scalar dequantisation q*scale + bias with
 *           the group index row*groups + col/64, little-endian BF16; the
 *           tied-embedding row it returns is computed in f32 and stored as
 *           f16),
 *        -- the f16 activations of the Metal GEMV (x and y are f16 there).
 *   [P4] fuel-transformers 0.19.1, src/models/lazy_quantized_whisper.rs
 *        -- module documentation (Q4_0 is ggml's BlockQ4_0 / from_float),
 *        -- quantize_in_out_to_q4_0 (row-major block stream, 18-byte
 *           blocks, zero padding to a 4-byte multiple, little-endian words),
 *        -- q_linear (matmul over the block stream; bias applied outside).
 *
 * Parity pins for every function here live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define QDO_GROUP 64 /* [P3] GROUP_SIZE: affine group width along K */
#define QDO_QK 32    /* [P4] QK4_0: elements per Q4_0 block          */
#define QDO_BLOCK 18 /* [P4] size_of::<BlockQ4_0>() == 18           */

/* ---- IEEE decoders ---------------------------------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * normal: (1024 + f) * 2^(e - 25); subnormal: f * 2^-24. */
double qdo_f16_to_f64(uint16_t h) {
  int sign = h >> 15;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* bfloat16: the upper half of a binary32 -- 1 sign bit, 8 exponent bits
 * (bias 127), 7 fraction bits.  normal: (128 + f) * 2^(e - 134);
 * subnormal: f * 2^-133. */
double qdo_bf16_to_f64(uint16_t b) {
  int sign = b >> 15;
  int e = (b >> 7) & 0xff;
  int f = b & 0x7f;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133);
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + f), e - 134);
  return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even, written from the
 * bit layouts (gradual underflow to subnormals, overflow to infinity). */
uint16_t qdo_f32_to_f16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t ex = (u >> 23) & 0xffu;
  uint32_t man = u & 0x7fffffu;
  if (ex == 0xff) /* infinity or NaN (NaN made quiet) */
    return (uint16_t)(sign | 0x7c00u | (man ? 0x200u : 0u));
  if (ex == 0) /* binary32 subnormal or zero: below half the least half */
    return sign;
  int e = (int)ex - 127;            /* value = m * 2^(e - 23)          */
  uint32_t m = man | 0x800000u;     /* 24-bit significand              */
  int qe = (e < -14) ? -24 : e - 10; /* exponent of one unit in the last place of the result */
  int shift = qe - (e - 23);        /* low bits of m below that unit   */
  if (shift > 24) /* m * 2^-shift < 1/2: rounds to zero */
    return sign;
  uint32_t q = m >> shift;
  uint32_t rem = m & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u)))
    q += 1u;
  if (qe == -24) /* subnormal range; q == 1024 is the least normal */
    return (uint16_t)(sign | q);
  if (q == 2048u) {
    q = 1024u;
    qe += 1;
  }
  int biased = qe + 25;
  if (biased >= 31)
    return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | ((uint32_t)biased << 10) | (q - 1024u));
}

/* binary32 -> bfloat16, round to nearest, ties to even: keep the upper 16
 * bits of the binary32 pattern, rounding on the lower 16 (NaN made quiet). */
uint16_t qdo_f32_to_bf16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu))
    return (uint16_t)((u >> 16) | 0x40u);
  uint32_t low = u & 0xffffu, keep = u >> 16;
  if (low > 0x8000u || (low == 0x8000u && (keep & 1u)))
    keep += 1u; /* a carry into the exponent is the correct rounding */
  return (uint16_t)keep;
}

/* ---- affine-INT8 g64 ---------------------------------------------------- */

/* Byte sizes and offsets of the single resident buffer
 * [codes | BF16 scales | BF16 biases]  ([P3] PackedLinear::resident). */
int64_t qdo_affine_scales_offset(int64_t rows, int64_t cols) { return rows * cols; }
int64_t qdo_affine_biases_offset(int64_t rows, int64_t cols) {
  return rows * cols + rows * (cols / QDO_GROUP) * 2;
}
int64_t qdo_affine_bytes(int64_t rows, int64_t cols) {
  return rows * cols + 2 * rows * (cols / QDO_GROUP) * 2;
}

/* [P3] load_packed_linear: blob = weight bytes, then scales, then biases. */
void qdo_affine_pack(const uint8_t *codes, const uint8_t *scales,
                     const uint8_t *biases, int64_t rows, int64_t cols,
                     uint8_t *blob) {
  int64_t companion = rows * (cols / QDO_GROUP) * 2;
  memcpy(blob, codes, (size_t)(rows * cols));
  memcpy(blob + rows * cols, scales, (size_t)companion);
  memcpy(blob + rows * cols + companion, biases, (size_t)companion);
}

static uint16_t le16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* One dequantised weight w[r, c] = q * scale + bias ([P3] embed_row_bytes):
 * code byte r*cols + c, group r*groups + c/64, BF16 little-endian. */
double qdo_affine_weight(const uint8_t *blob, int64_t rows, int64_t cols,
                         int64_t r, int64_t c) {
  int64_t groups = cols / QDO_GROUP;
  const uint8_t *scales = blob + qdo_affine_scales_offset(rows, cols);
  const uint8_t *biases = blob + qdo_affine_biases_offset(rows, cols);
  int64_t g = r * groups + c / QDO_GROUP;
  double q = (double)blob[r * cols + c];
  double s = qdo_bf16_to_f64(le16(scales + 2 * g));
  double b = qdo_bf16_to_f64(le16(biases + 2 * g));
  return q * s + b;
}

/* y[i, j] = sum_c w[row_sel[j], c] * x[m_sel[i], c], x [m, cols] row-major,
 * BF16 bits (x_f16 == 0) or f16 bits (x_f16 != 0).  Selections let large
 * shapes be checked on sampled outputs; pass NULL for "all". */
void qdo_affine_gemv(const uint8_t *blob, int64_t rows, int64_t cols,
                     const uint16_t *x_bits, int x_f16, int64_t m, const int64_t *m_sel,
                     int64_t n_m, const int64_t *row_sel, int64_t n_rows,
                     double *y) {
  if (!m_sel) n_m = m;
  if (!row_sel) n_rows = rows;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < n_rows; ++j) {
    int64_t r = row_sel ? row_sel[j] : j;
    for (int64_t i = 0; i < n_m; ++i) {
      int64_t t = m_sel ? m_sel[i] : i;
      double acc = 0.0;
      for (int64_t c = 0; c < cols; ++c)
        acc += qdo_affine_weight(blob, rows, cols, r, c) *
               (x_f16 ? qdo_f16_to_f64(x_bits[t * cols + c])
                      : qdo_bf16_to_f64(x_bits[t * cols + c]));
      y[i * n_rows + j] = acc;
    }
  }
}

/* y[j] = sum_c w(r, c) x[c] for one f64 input vector (rows row_sel[j], or
 * all rows): the same exact-weight dot product as qdo_affine_gemv for inputs
 * that are not 16-bit values (the unrounded decoder-step reference). */
void qdo_affine_gemv_f64(const uint8_t *blob, int64_t rows, int64_t cols, const double *x,
                         const int64_t *row_sel, int64_t n_rows, double *y) {
  if (!row_sel) n_rows = rows;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < n_rows; ++j) {
    int64_t r = row_sel ? row_sel[j] : j;
    double acc = 0.0;
    for (int64_t c = 0; c < cols; ++c) acc += qdo_affine_weight(blob, rows, cols, r, c) * x[c];
    y[j] = acc;
  }
}

/* [P3] embed_row_bytes: the tied-embedding row of `token` as 16-bit values,
 * each q*scale + bias evaluated in binary32 (q*scale is exact there: at most
 * 8 + 8 significant bits, so only the addition rounds) and then rounded to
 * f16 (out_f16 != 0, the page's store) or to BF16 -- two roundings, as the
 * page has them. */
void qdo_affine_embed_row(const uint8_t *blob, int64_t rows, int64_t cols,
                          int64_t token, int out_f16, uint16_t *out) {
  int64_t groups = cols / QDO_GROUP;
  const uint8_t *scales = blob + qdo_affine_scales_offset(rows, cols);
  const uint8_t *biases = blob + qdo_affine_biases_offset(rows, cols);
  for (int64_t c = 0; c < cols; ++c) {
    int64_t g = token * groups + c / QDO_GROUP;
    float q = (float)blob[token * cols + c];
    float s = (float)qdo_bf16_to_f64(le16(scales + 2 * g));
    float b = (float)qdo_bf16_to_f64(le16(biases + 2 * g));
    float v = q * s + b; /* -ffp-contract=off: a product, then a rounded sum */
    out[c] = out_f16 ? qdo_f32_to_f16_rne(v) : qdo_f32_to_bf16_rne(v);
  }
}

/* ---- ggml Q4_0 ----------------------------------------------------------- */

int64_t qdo_q4_0_bytes(int64_t rows, int64_t cols) {
  /* [P4] quantize_in_out_to_q4_0: 18 bytes per block, zero-padded up to a
   * multiple of 4 so the stream can be viewed as little-endian u32 words. */
  int64_t total = rows * (cols / QDO_QK) * QDO_BLOCK;
  return (total % 4) ? total + (4 - total % 4) : total;
}

/* One dequantised weight of the block stream: block (n, b) starts at byte
 * 18*(n*cols/32 + b); bytes 0..1 are the f16 delta d (little-endian); byte
 * 2+j holds element j in its low nibble and element j+16 in its high nibble;
 * w = d * (q - 8). */
double qdo_q4_0_weight(const uint8_t *wq, int64_t cols, int64_t n, int64_t k) {
  const uint8_t *blk = wq + QDO_BLOCK * (n * (cols / QDO_QK) + k / QDO_QK);
  int j = (int)(k % QDO_QK);
  double d = qdo_f16_to_f64(le16(blk));
  int q = (j < 16) ? (blk[2 + j] & 0x0f) : (blk[2 + j - 16] >> 4);
  return d * (double)(q - 8);
}

/* y[i, j] = sum_k w[row_sel[j], k] * x[m_sel[i], k].  x is f32 (x_kind 0)
 * or BF16 bits (x_kind 1), row-major [m, cols]. */
void qdo_q4_0_gemm(const uint8_t *wq, int64_t rows, int64_t cols,
                   const void *x, int x_kind, int64_t m, const int64_t *m_sel,
                   int64_t n_m, const int64_t *row_sel, int64_t n_rows,
                   double *y) {
  const float *xf = (const float *)x;
  const uint16_t *xb = (const uint16_t *)x;
  if (!m_sel) n_m = m;
  if (!row_sel) n_rows = rows;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < n_rows; ++j) {
    int64_t n = row_sel ? row_sel[j] : j;
    for (int64_t i = 0; i < n_m; ++i) {
      int64_t t = m_sel ? m_sel[i] : i;
      double acc = 0.0;
      for (int64_t k = 0; k < cols; ++k) {
        double xv = x_kind ? qdo_bf16_to_f64(xb[t * cols + k])
                           : (double)xf[t * cols + k];
        acc += qdo_q4_0_weight(wq, cols, n, k) * xv;
      }
      y[i * n_rows + j] = acc;
    }
  }
}

/* f32 -> Q4_0 encoder for one block of 32 values (ggml's Q4_0 reference
 * quantiser, which [P4] names as the bake's algorithm):
 *   1. find the element of largest magnitude, first index winning ties;
 *   2. d = that element / -8 and id = 1/d (0 when d is 0), in f32;
 *   3. each nibble is trunc(x*id + 8.5), both operations rounded to f32
 *      separately, clamped to at most 15;
 *   4. the block stores d as f16 (round to nearest even) and packs element
 *      j in the low and element j+16 in the high nibble of byte 2+j. */
static void qdo_q4_0_encode_block(const float *x, uint8_t *out) {
  float amax = 0.0f, mx = 0.0f;
  for (int j = 0; j < QDO_QK; ++j) {
    float a = fabsf(x[j]);
    if (a > amax) {
      amax = a;
      mx = x[j];
    }
  }
  float d = mx / -8.0f;
  float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  uint8_t q[QDO_QK];
  for (int j = 0; j < QDO_QK; ++j) {
    volatile float p = x[j] * id; /* rounded product ... */
    volatile float t = p + 8.5f;  /* ... then rounded sum: never fused */
    int qi;
    if (t != t)
      qi = 0; /* NaN input lies outside the contract; pinned to 0 */
    else if (t >= 15.0f)
      qi = 15;
    else if (t <= 0.0f)
      qi = 0;
    else
      qi = (int)t; /* truncation == floor for t > 0 */
    q[j] = (uint8_t)qi;
  }
  uint16_t hd = qdo_f32_to_f16_rne(d);
  out[0] = (uint8_t)(hd & 0xff);
  out[1] = (uint8_t)(hd >> 8);
  for (int j = 0; j < 16; ++j)
    out[2 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
}

/* [P4] quantize_in_out_to_q4_0 steps 2-3 for a row-major [rows, cols] f32
 * matrix (rows = out_features, cols = in_features, cols % 32 == 0): blocks
 * row-major, then zero bytes up to a multiple of 4.  Writes
 * qdo_q4_0_bytes(rows, cols) bytes. */
void qdo_q4_0_quantize(const float *w, int64_t rows, int64_t cols,
                       uint8_t *out) {
  int64_t nb = rows * (cols / QDO_QK);
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b)
    qdo_q4_0_encode_block(w + QDO_QK * b, out + QDO_BLOCK * b);
  int64_t total = nb * QDO_BLOCK;
  for (int64_t p = total; p < qdo_q4_0_bytes(rows, cols); ++p)
    out[p] = 0;
}
