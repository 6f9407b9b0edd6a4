// decoder_ops.hip -- the small ops of a Qwen3 decode step around the GEMVs.
//
// turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step
// encodes, per layer: encode_rms_norm_bf16w (the residual row x, a BF16
// weight), encode_rms_norm_bf16w_perhead (q and the new K cache row, in
// place), encode_rope_neox_subdim (rotate-half RoPE at `position` on q and
// the K row), encode_residual_add (x += delta) and encode_silu_mul
// (gate = silu(gate) * up).  Every buffer is f16.  Each op here computes in
// fp32 from the f16 inputs and rounds its result to f16 once, where the page
// stores it; two ops that the page runs back to back are fused where the
// intermediate is still rounded and stored exactly as the page stores it:
//   * residual add + the next RMSNorm (x is rounded to f16 and written back,
//     and the norm reads that f16 value);
//   * per-head RMSNorm + RoPE (the normed head is rounded to f16 before the
//     rotation) + the copy of the V row into the cache.
// These kernels serve the standalone entry points (and the last residual
// add of a step without logits); inside qwen3_step_run the same arithmetic
// runs as prologues of the GEMVs (affine_gemv.hip) and of the attention
// (attention.hip).  `position` is read from device memory, so a captured
// graph can be replayed token after token.
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kNormThreads = 256;
constexpr int kNormMaxChunks = 8;  // 4-element chunks per thread: n <= 8192

__device__ __forceinline__ float round_f16(float v) { return f16_to_f32(f32_to_f16(v)); }

__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / kWave; ++w) s += red[w];
  return s;
}

// a = x, or f16(x + delta) stored to x_out when delta is given (x_out may be
// x: each element is read and written by the same thread); then
// out = f16(a / sqrt(mean(a^2) + eps) * w) when w is given; one workgroup.
// advance (optional): *advance += 1 once everything else is issued.
__global__ __launch_bounds__(kNormThreads) void add_rmsnorm_kernel(
    const uint16_t *x_, const uint16_t *__restrict__ delta_, const uint16_t *__restrict__ w_,
    int n, float eps, uint16_t *__restrict__ out_, uint16_t *x_out, int *__restrict__ advance) {
  __shared__ float red[kNormThreads / kWave];
  const QD_GLOBAL uint16_t *x = gp(x_);
  const int t = threadIdx.x;
  const int chunks = n / 4;
  float v[kNormMaxChunks][4];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kNormMaxChunks; ++k) {
    const int c = t + k * kNormThreads;
    if (c < chunks) {
      const u32x2 xw = *(const QD_GLOBAL u32x2 *)(x + 4 * c);
      const uint32_t xe[2] = {xw.x, xw.y};
      uint32_t de[2] = {0u, 0u};
      if (delta_) {
        const u32x2 dw = *(const QD_GLOBAL u32x2 *)(gp(delta_) + 4 * c);
        de[0] = dw.x;
        de[1] = dw.y;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a = f16_to_f32((xe[e / 2] >> (16 * (e % 2))) & 0xffffu);
        if (delta_) a = round_f16(a + f16_to_f32((de[e / 2] >> (16 * (e % 2))) & 0xffffu));
        v[k][e] = a;
        ss = fmaf(a, a, ss);
      }
      if (delta_) {
        u32x2 st;
        st.x = (uint32_t)f32_to_f16(v[k][0]) | ((uint32_t)f32_to_f16(v[k][1]) << 16);
        st.y = (uint32_t)f32_to_f16(v[k][2]) | ((uint32_t)f32_to_f16(v[k][3]) << 16);
        *(QD_GLOBAL u32x2 *)(gp(x_out) + 4 * c) = st;
      }
    }
  }
  if (w_) {
    const float inv = 1.f / sqrtf(block_sum(ss, red) / (float)n + eps);
#pragma unroll
    for (int k = 0; k < kNormMaxChunks; ++k) {
      const int c = t + k * kNormThreads;
      if (c < chunks) {
        const u32x2 ww = *(const QD_GLOBAL u32x2 *)(gp(w_) + 4 * c);
        const uint32_t we[2] = {ww.x, ww.y};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = f32_to_f16(v[k][e] * inv * bf16_to_f32((we[e / 2] >> (16 * (e % 2))) & 0xffffu));
        u32x2 st;
        st.x = o[0] | (o[1] << 16);
        st.y = o[2] | (o[3] << 16);
        *(QD_GLOBAL u32x2 *)(gp(out_) + 4 * c) = st;
      }
    }
  }
  if (advance && t == 0) gp(advance)[0] += 1;
}

// One wave per head: heads query heads (in place in q), then kv_heads K
// heads (from k_src into cache row `position` of k_cache, V row copied from
// v_src to v_cache).  Lane l < d/2 holds the RoPE pair (l, l + d/2).
__global__ __launch_bounds__(kWave) void qk_norm_rope_kernel(
    uint16_t *__restrict__ q_, const uint16_t *__restrict__ k_src, const uint16_t *__restrict__ v_src,
    const uint16_t *__restrict__ q_w, const uint16_t *__restrict__ k_w, int heads, int kv_heads,
    int d, float eps, float theta, const int *__restrict__ pos_dev, int capacity,
    uint16_t *__restrict__ k_cache, uint16_t *__restrict__ v_cache, unsigned *__restrict__ err) {
  const int b = blockIdx.x, l = threadIdx.x;
  const int pos = gp(pos_dev)[0];
  if (pos < 0 || pos >= capacity) {
    if (b == 0 && l == 0) atomicOr(err, 1u);
    return;
  }
  const bool is_q = b < heads;
  const int head = is_q ? b : b - heads;
  const int half = d / 2;
  const QD_GLOBAL uint16_t *src = gp(is_q ? (const uint16_t *)q_ : k_src) + (size_t)head * d;
  const QD_GLOBAL uint16_t *w = gp(is_q ? q_w : k_w);
  const size_t row = (size_t)pos * kv_heads * d + (size_t)head * d;
  QD_GLOBAL uint16_t *dst = is_q ? gp(q_) + (size_t)head * d : gp(k_cache) + row;
  const bool on = l < half;
  float x1 = 0.f, x2 = 0.f;
  if (on) {
    x1 = f16_to_f32(src[l]);
    x2 = f16_to_f32(src[l + half]);
  }
  const float inv = 1.f / sqrtf(wave_sum(x1 * x1 + x2 * x2) / (float)d + eps);
  if (!on) return;
  // the normed head as the page stores it (f16), then the rotation
  const float n1 = round_f16(x1 * inv * bf16_to_f32(w[l]));
  const float n2 = round_f16(x2 * inv * bf16_to_f32(w[l + half]));
  const double ang = (double)pos * pow((double)theta, -2.0 * (double)l / (double)d);
  const float c = (float)cos(ang), s = (float)sin(ang);
  dst[l] = f32_to_f16(n1 * c - n2 * s);
  dst[l + half] = f32_to_f16(n2 * c + n1 * s);
  if (!is_q) {
    const QD_GLOBAL uint16_t *vs = gp(v_src) + (size_t)head * d;
    QD_GLOBAL uint16_t *vd = gp(v_cache) + row;
    vd[l] = vs[l];
    vd[l + half] = vs[l + half];
  }
}

// out[i] = f16(silu(gate[i]) * up[i]), silu(g) = g / (1 + e^-g); 4 per thread.
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t *__restrict__ gate,
                                                       const uint16_t *__restrict__ up,
                                                       uint16_t *__restrict__ out, int n) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= n / 4) return;
  const u32x2 gw = *(const QD_GLOBAL u32x2 *)(gp(gate) + 4 * c);
  const u32x2 uw = *(const QD_GLOBAL u32x2 *)(gp(up) + 4 * c);
  const uint32_t ge[2] = {gw.x, gw.y}, ue[2] = {uw.x, uw.y};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float g = f16_to_f32((ge[e / 2] >> (16 * (e % 2))) & 0xffffu);
    const float u = f16_to_f32((ue[e / 2] >> (16 * (e % 2))) & 0xffffu);
    o[e] = f32_to_f16(g / (1.f + expf(-g)) * u);
  }
  u32x2 st;
  st.x = o[0] | (o[1] << 16);
  st.y = o[2] | (o[3] << 16);
  *(QD_GLOBAL u32x2 *)(gp(out) + 4 * c) = st;
}

}  // namespace

hipError_t launch_add_rmsnorm(const uint16_t *x, const uint16_t *delta, const uint16_t *w, int n,
                              float eps, uint16_t *out, uint16_t *x_out, int *advance,
                              hipStream_t stream) {
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(1), dim3(kNormThreads), 0, stream, x, delta, w, n,
                     eps, out, x_out, advance);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(uint16_t *q, const uint16_t *k_src, const uint16_t *v_src,
                               const uint16_t *q_w, const uint16_t *k_w, int heads, int kv_heads,
                               int d, float eps, float theta, const int *pos_dev, int capacity,
                               uint16_t *k_cache, uint16_t *v_cache, unsigned *err,
                               hipStream_t stream) {
  hipLaunchKernelGGL(qk_norm_rope_kernel, dim3(heads + kv_heads), dim3(kWave), 0, stream, q,
                     k_src, v_src, q_w, k_w, heads, kv_heads, d, eps, theta, pos_dev, capacity,
                     k_cache, v_cache, err);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const uint16_t *gate, const uint16_t *up, uint16_t *out, int n,
                           hipStream_t stream) {
  const int chunks = n / 4;
  hipLaunchKernelGGL(silu_mul_kernel, dim3((chunks + 255) / 256), dim3(256), 0, stream, gate, up,
                     out, n);
  return hipGetLastError();
}

}  // namespace qd
