// q4_0_quantize.hip -- bit-exact f32 -> ggml Q4_0 bake on gfx950.
//
// fuel-transformers 0.19.1, lazy_quantized_whisper.rs -- module
// documentation (ggml's BlockQ4_0::from_float) and quantize_in_out_to_q4_0
// (block stream, zero pad, u32 view).  Per block of 32:
//   d  = (element of largest |x|, first index on ties) / -8      (f32)
//   id = 1/d correctly rounded, or 0 when d == 0
//   q  = min(15, trunc(fl(fl(x*id) + 8.5)))  -- two roundings, never fused
//   bytes: f16(d) round-to-nearest-even, little-endian; byte 2+j =
//   q_j | q_{j+16} << 4.
// This translation unit is compiled with -ffp-contract=off and uses the
// explicitly rounded __fmul_rn / __fadd_rn / __fdiv_rn so no step can be
// contracted or approximated.  Denormals are kept (no flush to zero).
//
// Layout on the chip: eight lanes own one block (4 floats each, so one
// 16-byte load per lane and 1 KiB of contiguous input per wave
// instruction); the max-magnitude search is an 8-lane reduction that keeps
// the lowest index on ties; lane k < 4 of a block packs output bytes
// 2+4k .. 5+4k.  A wave's 8 output blocks (144 contiguous bytes) are
// assembled in LDS and written as 36 aligned dwords.
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kBlocksPerWave = 8;

__device__ __forceinline__ uint32_t nibble(float x, float id) {
  const float t = __fadd_rn(__fmul_rn(x, id), 8.5f);
  // t lies in [0, 16.5] for finite input; NaN (outside the contract) -> 0
  if (!(t > 0.f)) return 0u;
  if (t >= 15.f) return 15u;
  return (uint32_t)(int)t;  // truncation
}

__global__ __launch_bounds__(kThreads) void q4_0_quantize_kernel(
    const float *__restrict__ w, int64_t n_blocks, uint8_t *__restrict__ out) {
  __shared__ uint32_t stage[kWaves][36];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int blk_in_wave = lane >> 3;  // 0..7
  const int sub = lane & 7;           // this lane holds elements 4*sub..4*sub+3
  uint8_t *st = (uint8_t *)stage[wave];

  const int64_t step = (int64_t)gridDim.x * kWaves * kBlocksPerWave;
  for (int64_t base = ((int64_t)blockIdx.x * kWaves + wave) * kBlocksPerWave;
       base < n_blocks; base += step) {
    const int64_t blk = base + blk_in_wave;
    const bool valid = blk < n_blocks;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) v = *(const float4 *)(w + blk * 32 + sub * 4);

    // largest |x| within this lane (first index wins), then across the 8 lanes
    float amax = 0.f, mx = 0.f;
    int idx = 1 << 30;
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = fabsf(e[k]);
      if (a > amax) { amax = a; mx = e[k]; idx = sub * 4 + k; }
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const float oa = __shfl_xor(amax, o, kWave);
      const float om = __shfl_xor(mx, o, kWave);
      const int oi = __shfl_xor(idx, o, kWave);
      if (oa > amax || (oa == amax && oi < idx)) { amax = oa; mx = om; idx = oi; }
    }
    // mx now is the first element of maximal magnitude (or +0.0 if none)
    const float d = __fdiv_rn(mx, -8.0f);
    const float id = (d != 0.f) ? __fdiv_rn(1.0f, d) : 0.f;
    const uint32_t q0 = nibble(e[0], id), q1 = nibble(e[1], id);
    const uint32_t q2 = nibble(e[2], id), q3 = nibble(e[3], id);
    const uint32_t mine = q0 | (q1 << 8) | (q2 << 16) | (q3 << 24);
    // lanes 0..3 of a block hold elements 0..15, lanes 4..7 elements 16..31
    const uint32_t other = __shfl_xor(mine, 4, kWave);
    const uint16_t dh = __builtin_bit_cast(uint16_t, (_Float16)d);

    // assemble 8 blocks x 18 bytes in LDS
    if (sub < 4) {
      const uint32_t packed = mine | (other << 4);
      uint8_t *o = st + blk_in_wave * 18 + 2 + sub * 4;
      o[0] = (uint8_t)packed;
      o[1] = (uint8_t)(packed >> 8);
      o[2] = (uint8_t)(packed >> 16);
      o[3] = (uint8_t)(packed >> 24);
    }
    if (sub == 0) {
      st[blk_in_wave * 18] = (uint8_t)dh;
      st[blk_in_wave * 18 + 1] = (uint8_t)(dh >> 8);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // write the wave's bytes: whole dwords when all 8 blocks exist
    const int64_t nvalid = n_blocks - base < 8 ? n_blocks - base : 8;
    if (nvalid == 8) {
      // 144 bytes at byte offset 18*base; base is a multiple of 8 so the
      // offset is a multiple of 144 and dword aligned
      if (lane < 36)
        ((uint32_t *)(out + 18 * base))[lane] = stage[wave][lane];
    } else {
      const int nbytes = (int)nvalid * 18;
      for (int i = lane; i < nbytes; i += kWave) out[18 * base + i] = st[i];
    }
    __builtin_amdgcn_wave_barrier();
  }
  // zero pad up to a multiple of 4 bytes (2 bytes when the count is odd)
  if (blockIdx.x == 0 && threadIdx.x == 0 && (n_blocks & 1)) {
    out[18 * n_blocks] = 0;
    out[18 * n_blocks + 1] = 0;
  }
}

}  // namespace

hipError_t launch_q4_0_quantize(const float *w, int64_t n_blocks, uint8_t *out,
                                hipStream_t stream) {
  const int64_t per_block = kWaves * kBlocksPerWave;
  int64_t grid = (n_blocks + per_block - 1) / per_block;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(q4_0_quantize_kernel, dim3((unsigned)grid), dim3(kThreads),
                     0, stream, w, n_blocks, out);
  return hipGetLastError();
}

}  // namespace qd
