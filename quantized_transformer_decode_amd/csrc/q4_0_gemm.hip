// q4_0_gemm.hip -- Q4_0 prefill GEMM on the gfx950 matrix cores.
//
// y[t, n] = sum_b d[n,b] * P[t,n,b],  P[t,n,b] = sum_j (q[n,b,j]-8) x[t,32b+j]
// (fuel-transformers 0.19.1, lazy_quantized_whisper.rs -- encoder_layer /
// q_linear run every projection over all encoder frames).  The integer codes
// (q - 8) in [-8, 7] are exact in BF16, so each 16x16x32 BF16 MFMA computes
// one block's partial product P exactly up to fp32 accumulation; the f16
// delta is applied to P in fp32 (rounding d*(q-8) to BF16 instead would cost
// up to 2^-9 relative error per weight).
//
// Tiling: a 256-thread workgroup owns a 64 (tokens) x 64 (weight rows) output
// tile; its four wavefronts each own 32 x 32 (2 x 2 MFMA tiles).  Each K step
// is one Q4_0 block (32 columns): x [64][32] BF16 and the dequantised codes
// [64][32] BF16 are staged in LDS, the deltas as fp32.
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 64;
constexpr int BN = 64;
constexpr int kLd = 40;  // LDS row stride in bf16 (32 + 8 pad, 80 bytes)

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

__global__ __launch_bounds__(kThreads) void q4_0_gemm_kernel(
    const uint8_t *__restrict__ w, int rows, int cols,
    const uint16_t *__restrict__ x, float *__restrict__ y, int m) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLd];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * kLd];
  __shared__ float Ds[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int bpr = cols >> 5;

  floatx4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < bpr; ++kb) {
    // x tile: 64 rows x 64 bytes; thread -> (row tid/4, 16-byte chunk tid%4)
    {
      const int r = tid >> 2, ch = tid & 3;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + r < m)
        v = *(const uint4 *)(x + (size_t)(m0 + r) * cols + kb * 32 + ch * 8);
      *(uint4 *)(As + r * kLd + ch * 8) = v;
    }
    // weight tile: threads 0..63 dequantise one block each
    if (tid < BN) {
      const int n = n0 + tid;
      uint32_t nib[4] = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
      float d = 0.f;
      if (n < rows) {
        const size_t flat = (size_t)n * bpr + kb;
        const size_t nb = 18 * flat + 2;
        const uint32_t *p = (const uint32_t *)(w + (nb & ~(size_t)3));
        const uint32_t sh = (uint32_t)(nb & 3);
        const uint32_t v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3];
        const uint32_t v4 = sh ? p[4] : 0u;
        nib[0] = __builtin_amdgcn_alignbyte(v1, v0, sh);
        nib[1] = __builtin_amdgcn_alignbyte(v2, v1, sh);
        nib[2] = __builtin_amdgcn_alignbyte(v3, v2, sh);
        nib[3] = __builtin_amdgcn_alignbyte(v4, v3, sh);
        d = f16_to_f32(*(const uint16_t *)(w + 18 * flat));
      }
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t v = nib[k];
        const float e0 = (float)((int)(v & 15u) - 8);
        const float e1 = (float)((int)((v >> 8) & 15u) - 8);
        const float e2 = (float)((int)((v >> 16) & 15u) - 8);
        const float e3 = (float)((int)((v >> 24) & 15u) - 8);
        const float f0 = (float)((int)((v >> 4) & 15u) - 8);
        const float f1 = (float)((int)((v >> 12) & 15u) - 8);
        const float f2 = (float)((int)((v >> 20) & 15u) - 8);
        const float f3 = (float)((int)((v >> 28) & 15u) - 8);
        lo[2 * k] = pack_bf16x2(e0, e1);
        lo[2 * k + 1] = pack_bf16x2(e2, e3);
        hi[2 * k] = pack_bf16x2(f0, f1);
        hi[2 * k + 1] = pack_bf16x2(f2, f3);
      }
      uint4 *dst = (uint4 *)(Bs + tid * kLd);
      dst[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);  // elements 0..7
      dst[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);  // 8..15
      dst[2] = make_uint4(hi[0], hi[1], hi[2], hi[3]);  // 16..23
      dst[3] = make_uint4(hi[4], hi[5], hi[6], hi[7]);  // 24..31
      Ds[tid] = d;
    }
    __syncthreads();

    const int kq = (lane >> 4) * 8;  // this lane's 8 K indices
    bf16x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 32 + i * 16 + (lane & 15);
      a[i] = *(const bf16x8 *)(As + r * kLd + kq);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = wn * 32 + j * 16 + (lane & 15);
      b[j] = *(const bf16x8 *)(Bs + c * kLd + kq);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float dj = Ds[wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const floatx4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            a[i], b[j], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        acc[i][j] += dj * p;
      }
    }
    __syncthreads();
  }

  // C layout of a 16x16 f32 MFMA tile: lane holds rows 4*(lane/16)+v of
  // column lane%16.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + v;
        if (t < m && n < rows) y[(size_t)t * rows + n] = acc[i][j][v];
      }
    }
}

}  // namespace

hipError_t launch_q4_0_gemm(const uint8_t *w, int rows, int cols,
                            const uint16_t *x, float *y, int m,
                            hipStream_t stream) {
  dim3 grid((rows + BN - 1) / BN, (m + BM - 1) / BM);
  hipLaunchKernelGGL(q4_0_gemm_kernel, grid, dim3(kThreads), 0, stream, w,
                     rows, cols, x, y, m);
  return hipGetLastError();
}

}  // namespace qd
