// qd_device.h -- small device helpers shared by the gfx950 kernels of
// libqdecode (bit-level conversions and wavefront reductions).  gfx950 only:
// wave64, 16x16x32 bf16 MFMA, hardware BF16 round-to-nearest-even convert.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qd {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// BF16 round-to-nearest-even (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
  return (float)h;
}

// Byte n (0..3) of a dword as float (v_cvt_f32_ubyteN).
template <int N>
__device__ __forceinline__ float ubyte(uint32_t v) {
  return (float)((v >> (8 * N)) & 0xffu);
}

// Sum over all 64 lanes of the wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum over aligned groups of W lanes (W = 2, 4, 8, 16, 32).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace qd
