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

// ---- batch 1: streaming kernel ---------------------------------------------
//
// Each wave owns a contiguous range of rows and walks its items -- (row,
// 1 KiB chunk) pairs, lane l holding bytes [16l, 16l+16) of the chunk -- in
// register groups of kG items, double-buffered: the next group's loads are
// issued (always the same number, so the compiler waits for exactly the
// group being consumed) before the current group is computed.  x sits in LDS
// in the xswz layout, fp32.

constexpr int kG = 8;
constexpr int kM1Threads = 512;
constexpr int kM1Waves = kM1Threads / kWave;

struct M1Group {
  uint4 q[kG];
  uint16_t sc[kG], bi[kG];
};

__device__ __forceinline__ void m1_issue(M1Group &g, const QD_GLOBAL uint8_t *w, int rows,
                                         int cols, int chunks, int lo, int n, int i0,
                                         int lane) {
  const int groups = cols >> 6;
  const QD_GLOBAL uint16_t *sc = (const QD_GLOBAL uint16_t *)(w + (size_t)rows * cols);
  int r = uni(i0 / chunks);
  int ch = uni(i0 - r * chunks);
  int row = lo + r;
#pragma unroll
  for (int k = 0; k < kG; ++k) {
    int col = ch * 1024 + lane * 16;
    if (col >= cols) col = 0;
    const u32x4 v =
        __builtin_nontemporal_load((const QD_GLOBAL u32x4 *)(w + (size_t)row * cols + col));
    g.q[k] = make_uint4(v.x, v.y, v.z, v.w);
    const size_t gi = (size_t)row * groups + (col >> 6);
    g.sc[k] = sc[gi];
    g.bi[k] = sc[(size_t)rows * groups + gi];
    if (i0 + k + 1 < n && ++ch == chunks) {
      ch = 0;
      ++row;
    }
  }
}

__device__ __forceinline__ void m1_compute(const M1Group &g, int cols, int chunks, int lo, int n,
                                           int i0, int lane, const float *xl,
                                           QD_GLOBAL uint16_t *y, float &rowsum) {
  int r = uni(i0 / chunks);
  int ch = uni(i0 - r * chunks);
  int row = lo + r;
  int xkey = -1;
  float4 x0, x1, x2, x3;
  float xs = 0.f;
#pragma unroll
  for (int k = 0; k < kG; ++k) {
    if (i0 + k < n) {
      const bool valid = ch * 1024 + lane * 16 < cols;
      if (ch != xkey) {  // x depends only on the chunk
        xkey = ch;
        const float *xp = xl + ch * 1024 + lane * 4;
        x0 = *(const float4 *)(xp);
        x1 = *(const float4 *)(xp + 256);
        x2 = *(const float4 *)(xp + 512);
        x3 = *(const float4 *)(xp + 768);
        xs = ((x0.x + x0.y) + (x0.z + x0.w)) + ((x1.x + x1.y) + (x1.z + x1.w)) +
             ((x2.x + x2.y) + (x2.z + x2.w)) + ((x3.x + x3.y) + (x3.z + x3.w));
      }
      float p = fmaf(bf16_to_f32(g.sc[k]), dot16(g.q[k], x0, x1, x2, x3),
                     bf16_to_f32(g.bi[k]) * xs);
      if (!valid) p = 0.f;
      rowsum += wave_sum_dpp(p);
      if (ch == chunks - 1) {
        if (lane == 0) y[row] = f32_to_bf16(rowsum);
        rowsum = 0.f;
      }
      if (++ch == chunks) {
        ch = 0;
        ++row;
      }
    }
  }
}

__global__ __launch_bounds__(kM1Threads) void affine_gemv_m1_kernel(
    const uint8_t *__restrict__ w_, int rows, int cols, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y_) {
  extern __shared__ __attribute__((aligned(16))) float xl[];  // chunks*1024, xswz layout
  const int chunks = (cols + 1023) >> 10;
  for (int e = threadIdx.x; e < cols; e += kM1Threads) xl[xswz(e)] = bf16_to_f32(x[e]);
  __syncthreads();
  const QD_GLOBAL uint8_t *w = gp(w_);
  QD_GLOBAL uint16_t *y = gp(y_);
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * kM1Waves;
  const int gw = blockIdx.x * kM1Waves + uni(threadIdx.x >> 6);
  const int lo = uni((int)(((int64_t)rows * gw) / nw));
  const int hi = uni((int)(((int64_t)rows * (gw + 1)) / nw));
  const int n = uni((hi - lo) * chunks);
  if (n == 0) return;
  float rowsum = 0.f;
  M1Group A, B;
  m1_issue(A, w, rows, cols, chunks, lo, n, 0, lane);
  for (int i = 0; i < n; i += 2 * kG) {
    m1_issue(B, w, rows, cols, chunks, lo, n, i + kG < n ? i + kG : i, lane);
    m1_compute(A, cols, chunks, lo, n, i, lane, xl, y, rowsum);
    if (i + kG >= n) break;
    m1_issue(A, w, rows, cols, chunks, lo, n, i + 2 * kG < n ? i + 2 * kG : i + kG, lane);
    m1_compute(B, cols, chunks, lo, n, i + kG, lane, xl, y, rowsum);
  }
}

}  // namespace

hipError_t launch_affine_gemv(const uint8_t *w, int rows, int cols,
                              const uint16_t *x, uint16_t *y, int m,
                              hipStream_t stream) {
  if (m == 1) {
    // waves: about two register groups of items each, at most 4 workgroups
    // of 8 waves per CU
    int cus = device_cus();
    if (cus < 1) cus = 256;
    const int64_t items = (int64_t)rows * ((cols + 1023) / 1024);
    int64_t wgs = (items + 2 * kG * kM1Waves - 1) / (2 * kG * kM1Waves);
    if (wgs > 4 * (int64_t)cus) wgs = 4 * (int64_t)cus;
    if (wgs < 1) wgs = 1;
    const size_t lds = (size_t)((cols + 1023) / 1024) * 1024 * 4;
    hipLaunchKernelGGL(affine_gemv_m1_kernel, dim3((unsigned)wgs), dim3(kM1Threads), lds,
                       stream, w, rows, cols, x, y);
    return hipGetLastError();
  }
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
