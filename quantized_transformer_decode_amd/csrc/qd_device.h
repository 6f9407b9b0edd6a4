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
typedef float floatx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// BF16 round-to-nearest-even (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// binary32 -> binary16, round to nearest even (v_cvt_f16_f32; f16
// subnormals are kept).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
  return (float)h;
}

// The q_linear epilogue: + bias[n] (when given), then the tanh form of GELU,
// 0.5 v (1 + tanh(z)) with z = sqrt(2/pi) (v + 0.044715 v^3), with gelu.
// Evaluated as v / (1 + e^(-2z)) (the same function: 0.5 (1 + tanh z) is
// the logistic function of 2z): one exponential and one reciprocal, a few
// ulp, with no cancellation (1 + e^(-2z) >= 1; for z -> -inf the
// reciprocal of infinity gives -0).  Against the library tanhf: the
// Whisper-large q_linear encoder layer at 1500 frames 0.167 -> 0.161 ms.
__device__ __forceinline__ float linear_epilogue(float v, const float *bias, int n, int gelu) {
  if (bias) v += ((const __attribute__((address_space(1))) float *)bias)[n];
  if (gelu) {
    const float z = 0.7978845608028654f * fmaf(0.044715f * v, v * v, v);
    v = v * __builtin_amdgcn_rcpf(1.f + __expf(-2.f * z));
  }
  return v;
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Pointers that are not kernel arguments are generic; casting them to the
// global address space makes their accesses global_* instructions (flat_*
// would also count against the LDS wait counter).
#define QD_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ QD_GLOBAL T *gp(T *p) {
  return (QD_GLOBAL T *)p;
}

// Wave-uniform value forced into a scalar register.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Sum over the 64 lanes with DPP row operations; the total ends in lane 63
// and is broadcast with readlane.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  int x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true));  // quad [1,0,3,2]
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true));  // quad [2,3,0,1]
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, true)); // row half mirror
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, true)); // row mirror
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false)); // row bcast 15
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false)); // row bcast 31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// 16 u8 codes (one 16-byte load) against 16 activations.
__device__ __forceinline__ float dot16(const uint4 q, const float4 a, const float4 b,
                                       const float4 c, const float4 d) {
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

// Eight u8 codes (two dwords, byte order) as an MFMA BF16 fragment: integers
// 0..255 are exact in BF16 (v_cvt_f32_ubyteN + v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 codes8_bf16(uint32_t a, uint32_t b) {
  const floatx8 f = {ubyte<0>(a), ubyte<1>(a), ubyte<2>(a), ubyte<3>(a),
                     ubyte<0>(b), ubyte<1>(b), ubyte<2>(b), ubyte<3>(b)};
  return __builtin_convertvector(f, bf16x8);
}

// The same as f16 (0..255 are exact in f16 too).
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ halfx8 codes8_f16(uint32_t a, uint32_t b) {
  const floatx8 f = {ubyte<0>(a), ubyte<1>(a), ubyte<2>(a), ubyte<3>(a),
                     ubyte<0>(b), ubyte<1>(b), ubyte<2>(b), ubyte<3>(b)};
  return __builtin_convertvector(f, halfx8);
}

// LDS layout of an activation vector for the wave-per-1KiB-chunk GEMVs:
// within each 1024-column chunk, column 16*l + 4*q + t (lane l's q-th float4)
// is stored at float (q*64 + l)*4 + t, so each of a wave's four float4
// reads is lane-contiguous (no bank conflicts).
__device__ __forceinline__ int xswz(int e) {
  const int chunk = e & ~1023, r = e & 1023;
  return chunk + ((((r >> 2) & 3) * 64 + (r >> 4)) << 2) + (r & 3);
}

// Sum over aligned groups of W lanes (W = 2, 4, 8, 16, 32).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace qd
