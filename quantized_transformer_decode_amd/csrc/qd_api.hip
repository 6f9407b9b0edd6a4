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

#include "../../include/qdecode.h"
#include "qd_internal.h"

namespace {

constexpr int64_t kMaxGemvCols = 8192;  // LDS copy of x per workgroup
constexpr int64_t kMaxGemmCols = 65536;
constexpr int64_t kMaxGemmM = int64_t(1) << 22;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

thread_local int g_last_hip = 0;

// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_arch[64];

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

}  // namespace

extern "C" {

const char *qd_status_string(int status) {
  switch (status) {
    case QD_OK: return "QD_OK";
    case QD_EINVAL: return "QD_EINVAL: invalid argument (null pointer, size out of range or overlapping buffers)";
    case QD_ESHAPE: return "QD_ESHAPE: matrix width violates the format's divisibility rule";
    case QD_EALIGN: return "QD_EALIGN: pointer not aligned as the kernel requires";
    case QD_EDEVICE: return "QD_EDEVICE: no current HIP device, or it is not gfx950";
    case QD_EHIP: return "QD_EHIP: the HIP runtime reported an error";
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

qd_status qgemv_affine_i8_g64(const void *w_packed, int64_t rows, int64_t cols,
                              const void *x_bf16, void *y_bf16, int64_t m,
                              void *stream) {
  if (!w_packed || !x_bf16 || !y_bf16) return QD_EINVAL;
  if (rows < 1 || rows > kMaxRows || m < 1 || m > 16 || cols < 1) return QD_EINVAL;
  if (cols % 64 != 0 || cols > kMaxGemvCols) return QD_ESHAPE;
  if (!aligned(w_packed, 16) || !aligned(x_bf16, 16) || !aligned(y_bf16, 2))
    return QD_EALIGN;
  const size_t ny = (size_t)m * rows * 2;
  if (overlap(y_bf16, ny, w_packed, affine_bytes(rows, cols)) ||
      overlap(y_bf16, ny, x_bf16, (size_t)m * cols * 2))
    return QD_EINVAL;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = qd::launch_affine_gemv((const uint8_t *)w_packed, (int)rows,
                                        (int)cols, (const uint16_t *)x_bf16,
                                        (uint16_t *)y_bf16, (int)m,
                                        (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

qd_status qgemv_q4_0(const void *w_q4_0, int64_t rows, int64_t cols,
                     const float *x, float *y, int64_t m, void *stream) {
  if (!w_q4_0 || !x || !y) return QD_EINVAL;
  if (rows < 1 || rows > kMaxRows || m < 1 || m > 16 || cols < 1) return QD_EINVAL;
  if (cols % 256 != 0 || cols > kMaxGemvCols) return QD_ESHAPE;
  if (!aligned(w_q4_0, 16) || !aligned(x, 16) || !aligned(y, 4)) return QD_EALIGN;
  const size_t ny = (size_t)m * rows * 4;
  if (overlap(y, ny, w_q4_0, q40_bytes(rows, cols)) ||
      overlap(y, ny, x, (size_t)m * cols * 4))
    return QD_EINVAL;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = qd::launch_q4_0_gemv((const uint8_t *)w_q4_0, (int)rows,
                                      (int)cols, x, y, (int)m,
                                      (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
}

qd_status qgemm_q4_0_prefill(const void *w_q4_0, int64_t rows, int64_t cols,
                             const void *x_bf16, float *y, int64_t m,
                             void *stream) {
  if (!w_q4_0 || !x_bf16 || !y) return QD_EINVAL;
  if (rows < 1 || rows > kMaxRows || m < 1 || m > kMaxGemmM || cols < 1) return QD_EINVAL;
  if (cols % 256 != 0 || cols > kMaxGemmCols) return QD_ESHAPE;
  if (!aligned(w_q4_0, 16) || !aligned(x_bf16, 16) || !aligned(y, 16))
    return QD_EALIGN;
  const size_t ny = (size_t)m * rows * 4;
  if (overlap(y, ny, w_q4_0, q40_bytes(rows, cols)) ||
      overlap(y, ny, x_bf16, (size_t)m * cols * 2))
    return QD_EINVAL;
  qd_status st = check_device();
  if (st != QD_OK) return st;
  hipError_t e = qd::launch_q4_0_gemm((const uint8_t *)w_q4_0, (int)rows,
                                      (int)cols, (const uint16_t *)x_bf16, y,
                                      (int)m, (hipStream_t)stream);
  return e == hipSuccess ? QD_OK : hip_fail(e);
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

}  // extern "C"
