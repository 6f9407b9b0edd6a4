// q4_0_gemv.hip -- ggml Q4_0 dequant GEMV for gfx950, M <= 16 rows, f32.
//
// y[t, n] = sum_b d[n,b] * (sum_j q[n,b,j] * x[t,32b+j] - 8 * X[t,b])
// with X[t,b] the sum of x over block b: the "-8" of w = d*(q-8)
// (fuel-transformers 0.19.1, lazy_quantized_whisper.rs -- module
// documentation / quantize_in_out_to_q4_0 for the block format, q_linear for
// the matmul) is folded into one multiply-add per block.
//
// Layout on the chip: eight lanes share an output row and walk its blocks
// b = sub, sub+8, ...; eight lanes therefore read 8 consecutive 18-byte
// blocks (144 contiguous bytes) per load.  A block's 16 nibble bytes start
// at byte 18*flat+2, which is 4-byte aligned for odd flat block indices and
// 2 bytes off for even ones; the lane reads the enclosing dwords and
// realigns them with v_alignbyte_b32.  Each lane handles R rows at once so
// the 32 x values it reads from LDS serve R blocks.
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kLdsBudget = 64 * 1024;

__device__ __forceinline__ float nib_dot8(uint32_t v, const float *xp) {
  // v holds elements j..j+3 (low nibbles) and j+16..j+19 (high nibbles)
  const uint32_t lo = v & 0x0f0f0f0fu;
  const uint32_t hi = (v >> 4) & 0x0f0f0f0fu;
  float s = ubyte<0>(lo) * xp[0];
  s = fmaf(ubyte<1>(lo), xp[1], s);
  s = fmaf(ubyte<2>(lo), xp[2], s);
  s = fmaf(ubyte<3>(lo), xp[3], s);
  s = fmaf(ubyte<0>(hi), xp[16], s);
  s = fmaf(ubyte<1>(hi), xp[17], s);
  s = fmaf(ubyte<2>(hi), xp[18], s);
  s = fmaf(ubyte<3>(hi), xp[19], s);
  return s;
}

template <int MT, int R>
__global__ __launch_bounds__(kThreads) void q4_0_gemv_kernel(
    const uint8_t *__restrict__ w, int rows, int cols,
    const float *__restrict__ x, float *__restrict__ y, int t0, int m) {
  extern __shared__ float lds[];
  const int bpr = cols >> 5;
  float *xs = lds;                // [MT][cols]
  float *xsum = lds + MT * cols;  // [MT][cols/32]
  for (int i = threadIdx.x; i < MT * cols; i += kThreads) {
    const int t = i / cols;
    const int c = i - t * cols;
    xs[i] = (t0 + t < m) ? x[(size_t)(t0 + t) * cols + c] : 0.f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < MT * bpr; i += kThreads) {
    const float *p = xs + (size_t)i * 32;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) s += p[k];
    xsum[i] = s;
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int sg = lane >> 3;
  const int sub = lane & 7;
  const int rows_per_wave = 8 * R;

  for (int row0 = (blockIdx.x * kWaves + wave) * rows_per_wave; row0 < rows;
       row0 += gridDim.x * kWaves * rows_per_wave) {
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[r][t] = 0.f;

    for (int b = sub; b < bpr; b += 8) {
      uint32_t nib[R][4];
      float d[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = row0 + sg * R + r;
        if (n < rows) {
          const size_t flat = (size_t)n * bpr + b;
          const size_t nb = 18 * flat + 2;
          const uint32_t *p = (const uint32_t *)(w + (nb & ~(size_t)3));
          const uint32_t sh = (uint32_t)(nb & 3);  // 0 or 2
          const uint32_t v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3];
          // Only the 2-byte-offset case needs the fifth dword; it lies inside
          // the stream (the next block, or the pad of an odd block count).
          const uint32_t v4 = sh ? p[4] : 0u;
          nib[r][0] = __builtin_amdgcn_alignbyte(v1, v0, sh);
          nib[r][1] = __builtin_amdgcn_alignbyte(v2, v1, sh);
          nib[r][2] = __builtin_amdgcn_alignbyte(v3, v2, sh);
          nib[r][3] = __builtin_amdgcn_alignbyte(v4, v3, sh);
          d[r] = f16_to_f32(*(const uint16_t *)(w + 18 * flat));
        } else {
          nib[r][0] = nib[r][1] = nib[r][2] = nib[r][3] = 0x88888888u;
          d[r] = 0.f;
        }
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const float *xp = xs + t * cols + 32 * b;
        const float xb = xsum[t * bpr + b];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float s = nib_dot8(nib[r][0], xp);
          s += nib_dot8(nib[r][1], xp + 4);
          s += nib_dot8(nib[r][2], xp + 8);
          s += nib_dot8(nib[r][3], xp + 12);
          acc[r][t] = fmaf(d[r], fmaf(-8.f, xb, s), acc[r][t]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const float v = group_sum<8>(acc[r][t]);
        const int n = row0 + sg * R + r;
        if (sub == 0 && n < rows && t0 + t < m)
          y[(size_t)(t0 + t) * rows + n] = v;
      }
  }
}

template <int MT, int R>
hipError_t launch_pass(const uint8_t *w, int rows, int cols, const float *x,
                       float *y, int t0, int m, hipStream_t stream) {
  const size_t lds = (size_t)MT * cols * 4 + (size_t)MT * (cols / 32) * 4;
  const int per_block = kWaves * 8 * R;
  int grid = (rows + per_block - 1) / per_block;
  if (grid > 2048) grid = 2048;
  hipLaunchKernelGGL((q4_0_gemv_kernel<MT, R>), dim3(grid), dim3(kThreads),
                     lds, stream, w, rows, cols, x, y, t0, m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q4_0_gemv(const uint8_t *w, int rows, int cols,
                            const float *x, float *y, int m,
                            hipStream_t stream) {
  const int cap = kLdsBudget / (cols * 4 + cols / 8);
  int t0 = 0;
  while (t0 < m) {
    const int left = m - t0;
    const int lim = left < cap ? left : cap;
    hipError_t e;
    int mt;
    if (lim >= 8) { mt = 8; e = launch_pass<8, 1>(w, rows, cols, x, y, t0, m, stream); }
    else if (lim >= 4) { mt = 4; e = launch_pass<4, 1>(w, rows, cols, x, y, t0, m, stream); }
    else if (lim >= 2) { mt = 2; e = launch_pass<2, 2>(w, rows, cols, x, y, t0, m, stream); }
    else { mt = 1; e = launch_pass<1, 2>(w, rows, cols, x, y, t0, m, stream); }
    if (e != hipSuccess) return e;
    t0 += mt;
  }
  return hipSuccess;
}

}  // namespace qd
