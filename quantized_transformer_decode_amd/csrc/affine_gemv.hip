// affine_gemv.hip -- affine-INT8 g64 dequant GEMV for gfx950, M <= 16 rows.
//
// Computes y[t, r] = sum_c (q[r,c] * s[r,c/64] + b[r,c/64]) * x[t,c]
// (turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- embed_row_bytes for the
// dequantisation, Qwen3AsrMetalEngine::gemv for the GEMV), regrouped as
//   y[t, r] = sum_{16-col chunk j} s * (sum_{c in j} q*x) + b * X[t, j]
// where X[t, j] is the sum of x over chunk j (a 16-column chunk never
// straddles a 64-column group).  Codes are exact in fp32, accumulation is
// fp32, the output is rounded once to BF16 (nearest even).
//
// Layout on the chip: one wavefront streams R rows at a time; lane l reads
// the 16-byte code chunks l, l+64, ... of each row (a full 1 KiB of one row
// per load instruction, fully coalesced), converts the bytes with
// v_cvt_f32_ubyteN and multiplies against x, which every workgroup stages
// once in LDS as fp32 together with the per-chunk sums X.
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kLdsBudget = 64 * 1024;

__device__ __forceinline__ float dot16(const uint4 q, const float4 a,
                                       const float4 b, const float4 c,
                                       const float4 d) {
  float s = ubyte<0>(q.x) * a.x;
  s = fmaf(ubyte<1>(q.x), a.y, s);
  s = fmaf(ubyte<2>(q.x), a.z, s);
  s = fmaf(ubyte<3>(q.x), a.w, s);
  s = fmaf(ubyte<0>(q.y), b.x, s);
  s = fmaf(ubyte<1>(q.y), b.y, s);
  s = fmaf(ubyte<2>(q.y), b.z, s);
  s = fmaf(ubyte<3>(q.y), b.w, s);
  s = fmaf(ubyte<0>(q.z), c.x, s);
  s = fmaf(ubyte<1>(q.z), c.y, s);
  s = fmaf(ubyte<2>(q.z), c.z, s);
  s = fmaf(ubyte<3>(q.z), c.w, s);
  s = fmaf(ubyte<0>(q.w), d.x, s);
  s = fmaf(ubyte<1>(q.w), d.y, s);
  s = fmaf(ubyte<2>(q.w), d.z, s);
  s = fmaf(ubyte<3>(q.w), d.w, s);
  return s;
}

// Tokens t0 .. t0+MT-1 (those < m) against all rows.
template <int MT, int R>
__global__ __launch_bounds__(kThreads) void affine_gemv_kernel(
    const uint8_t *__restrict__ w, int rows, int cols,
    const uint16_t *__restrict__ x, uint16_t *__restrict__ y, int t0, int m) {
  extern __shared__ float lds[];
  float *xs = lds;                 // [MT][cols]
  float *xsum = lds + MT * cols;   // [MT][cols/16]
  const int nch = cols >> 4;
  for (int i = threadIdx.x; i < MT * cols; i += kThreads) {
    const int t = i / cols;
    const int c = i - t * cols;
    xs[i] = (t0 + t < m) ? bf16_to_f32(x[(size_t)(t0 + t) * cols + c]) : 0.f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < MT * nch; i += kThreads) {
    const float *p = xs + (size_t)i * 16;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += p[k];
    xsum[i] = s;
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int groups = cols >> 6;
  const uint16_t *scales = (const uint16_t *)(w + (size_t)rows * cols);
  const uint16_t *biases = scales + (size_t)rows * groups;

  for (int row0 = (blockIdx.x * kWaves + wave) * R; row0 < rows;
       row0 += gridDim.x * kWaves * R) {
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[r][t] = 0.f;

    for (int u = lane; u < nch; u += kWave) {
      uint4 q[R];
      float s[R], b[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = row0 + r;
        if (row < rows) {
          q[r] = *(const uint4 *)(w + (size_t)row * cols + 16 * u);
          const size_t g = (size_t)row * groups + (u >> 2);
          s[r] = bf16_to_f32(scales[g]);
          b[r] = bf16_to_f32(biases[g]);
        } else {
          q[r] = make_uint4(0, 0, 0, 0);
          s[r] = 0.f;
          b[r] = 0.f;
        }
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const float4 *xp = (const float4 *)(xs + t * cols + 16 * u);
        const float4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
        const float xc = xsum[t * nch + u];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float d = dot16(q[r], x0, x1, x2, x3);
          acc[r][t] = fmaf(s[r], d, fmaf(b[r], xc, acc[r][t]));
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const float v = wave_sum(acc[r][t]);
        if (lane == 0 && row0 + r < rows && t0 + t < m)
          y[(size_t)(t0 + t) * rows + row0 + r] = f32_to_bf16(v);
      }
  }
}

template <int MT, int R>
hipError_t launch_pass(const uint8_t *w, int rows, int cols, const uint16_t *x,
                       uint16_t *y, int t0, int m, hipStream_t stream) {
  const size_t lds = (size_t)MT * cols * 4 + (size_t)MT * (cols / 16) * 4;
  const int per_block = kWaves * R;
  int grid = (rows + per_block - 1) / per_block;
  if (grid > 2048) grid = 2048;
  hipLaunchKernelGGL((affine_gemv_kernel<MT, R>), dim3(grid), dim3(kThreads),
                     lds, stream, w, rows, cols, x, y, t0, m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_affine_gemv(const uint8_t *w, int rows, int cols,
                              const uint16_t *x, uint16_t *y, int m,
                              hipStream_t stream) {
  // Tokens per pass limited by the LDS copy of x (fp32 plus chunk sums).
  const int cap = kLdsBudget / (cols * 4 + cols / 4);
  int t0 = 0;
  while (t0 < m) {
    const int left = m - t0;
    const int lim = left < cap ? left : cap;
    hipError_t e;
    int mt;
    if (lim >= 16) { mt = 16; e = launch_pass<16, 1>(w, rows, cols, x, y, t0, m, stream); }
    else if (lim >= 8) { mt = 8; e = launch_pass<8, 1>(w, rows, cols, x, y, t0, m, stream); }
    else if (lim >= 4) { mt = 4; e = launch_pass<4, 2>(w, rows, cols, x, y, t0, m, stream); }
    else if (lim >= 2) { mt = 2; e = launch_pass<2, 4>(w, rows, cols, x, y, t0, m, stream); }
    else { mt = 1; e = launch_pass<1, 4>(w, rows, cols, x, y, t0, m, stream); }
    if (e != hipSuccess) return e;
    t0 += mt;
  }
  return hipSuccess;
}

}  // namespace qd
