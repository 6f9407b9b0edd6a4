// q4_0_gemm.hip -- Q4_0 prefill GEMM on the gfx950 matrix cores.
//
// y[t, n] = sum_b d[n,b] * P[t,n,b],  P[t,n,b] = sum_j (q[n,b,j]-8) x[t,32b+j]
// (fuel-transformers 0.19.1, lazy_quantized_whisper.rs -- encoder_layer /
// q_linear run every projection over all encoder frames).  The integer codes
// (q - 8) in [-8, 7] are exact in BF16, so each 16x16x32 BF16 MFMA computes
// one block's partial product P exactly up to fp32 accumulation; the f16
// delta is applied to P in fp32 (rounding d*(q-8) to BF16 instead would cost
// up to 2^-9 relative error per weight).  One fp32 multiply-add per output
// per block is exactly the VALU rate that matches the MFMA rate, so the
// kernel interleaves the MFMAs of block b with the delta scaling of block
// b-1's partial products.
//
// Up to four products that share x go in one launch (the q/k/v of a layer,
// 3 x 1280 output columns instead of 1280): their column tiles are numbered
// back to back and each workgroup looks up its matrix.  The q_linear
// epilogue (f32 bias, gelu_tanh for fc1) is applied at the store.
//
// Tiling: a 256-thread workgroup owns a BM (frames) x BN (weight rows)
// output tile, 64 x 64 by default; its four waves are 2 x 2, each
// BM/2 x BN/2.  Each LDS stage covers 128 columns of K (four Q4_0 blocks):
// x [BM][128] BF16 and the dequantised codes [BN][128] BF16, rows padded by
// 16 bytes so the 16 rows a fragment read touches fall in different banks;
// the deltas [BN][4] fp32.  Stages are double-buffered: the global loads of
// stage s+1 are in flight while stage s is computed.  64 x 64 tiles give
// ~2 workgroups per CU on a 1500 x 1280 output (the LDS, 70 KiB per
// workgroup, allows two) -- larger tiles leave the chip underfilled at
// Whisper-large shapes and smaller ones repeat the dequantisation.
#include "qd_device.h"
#include "qd_internal.h"

#ifndef QD_GEMM_BM
#define QD_GEMM_BM 64
#define QD_GEMM_BN 64
#endif

namespace qd {
namespace {

constexpr int kThreads = 256;
#ifndef QD_GEMM_BK
#define QD_GEMM_BK 128
#endif
constexpr int BK = QD_GEMM_BK;          // K columns per stage
constexpr int NB = BK / 32;             // Q4_0 blocks per stage
constexpr int CPR = BK / 8;             // 16-byte x chunks per tile row per stage
constexpr int LDA = BK + 8;             // LDS row stride in bf16

template <int BM, int BN>
struct Tile {
  static constexpr int A_ELEMS = BM * LDA;
  static constexpr int B_ELEMS = BN * LDA;
  static constexpr int STAGE_BYTES = (A_ELEMS + B_ELEMS) * 2 + BN * NB * 4;
  static constexpr int TM = BM / 32;    // 16x16 MFMA tiles per wave along M
  static constexpr int TN = BN / 32;    // ... along N (waves are 2 x 2)
  static constexpr int XCH = BM * CPR / kThreads;  // x 16-byte chunks per thread
  static constexpr int WB = BN * NB / kThreads;   // weight blocks per thread (<= 1)
};

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

// (q - 8) of four nibbles (one nibble per byte of `v`, bytes in element
// order) as four BF16 in two dwords: small integers are exact in BF16.
__device__ __forceinline__ u32x2v codes4_bf16(uint32_t v) {
  const floatx4 f = {ubyte<0>(v) - 8.f, ubyte<1>(v) - 8.f, ubyte<2>(v) - 8.f,
                     ubyte<3>(v) - 8.f};
  return __builtin_bit_cast(u32x2v, __builtin_convertvector(f, bf16x4));
}

template <int BM, int BN>
struct Stage {
  uint4 xa[Tile<BM, BN>::XCH];  // this thread's x chunks (16 bytes each)
  uint32_t w[5];                // this thread's Q4_0 block window
  uint32_t fb;                  // flat index parity | 2 if the row is past the end
  bool has_w;                   // this thread loads a weight block
};

// Global loads of one stage: x rows m0.., columns k0..k0+127; the weight
// block (row n0 + tid/NB, block kb0 + tid%NB).
template <int BM, int BN>
__device__ __forceinline__ void stage_load(Stage<BM, BN> &st, const QD_GLOBAL uint16_t *x,
                                           const QD_GLOBAL uint8_t *w, int m, int rows,
                                           int cols, int m0, int n0, int kb0, int tid) {
#pragma unroll
  for (int i = 0; i < Tile<BM, BN>::XCH; ++i) {
    const int c = tid + i * kThreads;  // 16-byte chunk of the BM x 2*BK-byte tile
    const int r = c / CPR, ch = c % CPR;
    // frames past m read frame m-1: they only feed output rows that are
    // never stored
    const int row = min(m0 + r, m - 1);
    const u32x4 v = *(const QD_GLOBAL u32x4 *)(x + (size_t)row * cols + kb0 * 32 + ch * 8);
    st.xa[i] = make_uint4(v.x, v.y, v.z, v.w);
  }
  st.has_w = tid < BN * NB;
  const int r = (tid / NB) % BN, b = tid % NB;
  int n = n0 + r;
  if (n >= rows) n = rows - 1;  // clamped rows are zeroed at the store
  const size_t flat = (size_t)n * (cols >> 5) + kb0 + b;
  // 20-byte window holding the block's 18 bytes: starts 2 bytes early for
  // odd flat indices (still inside the previous block) and on the block for
  // even ones (the 2 bytes past it exist: an even block is never the last
  // one, the block count per row being a multiple of 8)
  const QD_GLOBAL uint32_t *p =
      (const QD_GLOBAL uint32_t *)(w + 18 * flat - 2 * (flat & 1));
#pragma unroll
  for (int i = 0; i < 5; ++i) st.w[i] = p[i];
  st.fb = (uint32_t)(flat & 1) | (n0 + r >= rows ? 2u : 0u);
}

template <int BM, int BN>
__device__ __forceinline__ void stage_store(const Stage<BM, BN> &st, uint16_t *As, uint16_t *Bs,
                                            float *Ds, int tid) {
#pragma unroll
  for (int i = 0; i < Tile<BM, BN>::XCH; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / CPR, ch = c % CPR;
    *(uint4 *)(As + r * LDA + ch * 8) = st.xa[i];
  }
  if (!st.has_w) return;
  const int r = tid / NB, b = tid % NB;
  const bool odd = st.fb & 1, dead = st.fb & 2;
  // d: bytes 0-1 of the block; nibble bytes 2..17
  const uint32_t dbits = odd ? (st.w[0] >> 16) : (st.w[0] & 0xffffu);
  uint32_t nib[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    nib[k] = odd ? st.w[k + 1] : __builtin_amdgcn_alignbyte(st.w[k + 1], st.w[k], 2);
  uint32_t lo[8], hi[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // dword k: elements 4k..4k+3 in the low nibbles, 16+4k.. in the high
    const uint32_t v = dead ? 0x88888888u : nib[k];
    const u32x2v cl = codes4_bf16(v & 0x0f0f0f0fu), ch = codes4_bf16((v >> 4) & 0x0f0f0f0fu);
    lo[2 * k] = cl.x;
    lo[2 * k + 1] = cl.y;
    hi[2 * k] = ch.x;
    hi[2 * k + 1] = ch.y;
  }
  uint4 *dst = (uint4 *)(Bs + r * LDA + b * 32);
  dst[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);  // elements 0..7
  dst[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);  // 8..15
  dst[2] = make_uint4(hi[0], hi[1], hi[2], hi[3]);  // 16..23
  dst[3] = make_uint4(hi[4], hi[5], hi[6], hi[7]);  // 24..31
  Ds[r * NB + b] = dead ? 0.f : f16_to_f32(dbits);
}

template <int BM, int BN, bool MULTI, bool EPI>
__global__ __launch_bounds__(kThreads) void q4_0_gemm_kernel(
    const Q40Group grp, int cols, const uint16_t *__restrict__ x_, int m) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // this workgroup's matrix: column tiles are numbered back to back (a
  // single matrix takes its descriptor at fixed offsets)
  const int bx = blockIdx.x;
  int k = 0;
  if constexpr (MULTI) {
#pragma unroll
    for (int i = 1; i < kMaxGroup; ++i)
      if (i < grp.n && bx >= grp.tile0[i]) k = i;
    k = uni(k);
  }
  const QD_GLOBAL uint8_t *w = gp(grp.w[k]);
  const int rows = grp.rows[k];
  QD_GLOBAL float *y = gp(grp.y[k]);
  const float *bias = grp.bias[k];
  const QD_GLOBAL uint16_t *x = gp(x_);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = (bx - grp.tile0[k]) * BN;
  const int nstages = cols / BK;

  using T = Tile<BM, BN>;
  constexpr int TM = T::TM, TN = T::TN;
  auto As = [&](int buf) { return (uint16_t *)(smem + buf * T::STAGE_BYTES); };
  auto Bs = [&](int buf) { return (uint16_t *)(smem + buf * T::STAGE_BYTES) + T::A_ELEMS; };
  auto Ds = [&](int buf) {
    return (float *)(smem + buf * T::STAGE_BYTES + (T::A_ELEMS + T::B_ELEMS) * 2);
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int kq = (lane >> 4) * 8;  // this lane's 8 K indices within a block
  const int arow = wm * (BM / 2) + (lane & 15);
  const int bcol = wn * (BN / 2) + (lane & 15);
  // the bias of this lane's output columns, loaded before the K loop
  float bj[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + bcol + j * 16;
    bj[j] = (EPI && bias && n < rows) ? ((const QD_GLOBAL float *)bias)[n] : 0.f;
  }

  // One stage from LDS buffer `buf`: per block, TM x TN MFMAs of the exact
  // codes, then the previous block's partial products scaled by its deltas.
  auto compute = [&](int buf) {
    const uint16_t *A = As(buf);
    const uint16_t *Bm = Bs(buf);
    const float *D = Ds(buf);
    floatx4 p[2][TM][TN];  // partial products of two blocks in flight
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const bf16x8 *)(A + (arow + i * 16) * LDA + b * 32 + kq);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *(const bf16x8 *)(Bm + (bcol + j * 16) * LDA + b * 32 + kq);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          p[b & 1][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              af[i], bfr[j], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      if (b > 0) {  // scale the previous block while this block's MFMAs run
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const float dj = D[(bcol + j * 16) * NB + (b - 1)];
#pragma unroll
          for (int i = 0; i < TM; ++i) acc[i][j] += dj * p[(b - 1) & 1][i][j];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float dj = D[(bcol + j * 16) * NB + (NB - 1)];
#pragma unroll
      for (int i = 0; i < TM; ++i) acc[i][j] += dj * p[(NB - 1) & 1][i][j];
    }
  };

  // Double-buffered: the global loads of stage s+1 are in flight while stage
  // s is computed from LDS, then go to the other LDS buffer.
  Stage<BM, BN> st;
  stage_load(st, x, w, m, rows, cols, m0, n0, 0, tid);
  stage_store(st, As(0), Bs(0), Ds(0), tid);
  __syncthreads();
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstages) stage_load(st, x, w, m, rows, cols, m0, n0, (s + 1) * NB, tid);
    compute(buf);
    if (s + 1 < nstages) stage_store(st, As(buf ^ 1), Bs(buf ^ 1), Ds(buf ^ 1), tid);
    __syncthreads();
  }

  // C layout of a 16x16 f32 MFMA tile: lane holds rows 4*(lane/16)+v of
  // column lane%16.
  auto store = [&](auto act) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + bcol + j * 16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = m0 + wm * (BM / 2) + i * 16 + (lane >> 4) * 4 + v;
          if (t < m && n < rows)
            y[(size_t)t * rows + n] = EPI ? act(acc[i][j][v] + bj[j]) : acc[i][j][v];
        }
      }
  };
  if (EPI && grp.gelu)
    store([](float v) { return linear_epilogue(v, nullptr, 0, 1); });
  else
    store([](float v) { return v; });
}

template <int BM, int BN, bool MULTI, bool EPI>
hipError_t launch_tile(Q40Group g, int cols, const uint16_t *x, int m, hipStream_t stream) {
  const size_t lds = 2 * (size_t)Tile<BM, BN>::STAGE_BYTES;
  static bool attr_set = false;  // the limit is per function; setting it twice is harmless
  if (!attr_set && lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void *)q4_0_gemm_kernel<BM, BN, MULTI, EPI>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  g.tile0[0] = 0;
  for (int k = 0; k < g.n; ++k) g.tile0[k + 1] = g.tile0[k] + (g.rows[k] + BN - 1) / BN;
  for (int k = g.n; k < kMaxGroup; ++k) g.tile0[k + 1] = g.tile0[g.n];
  dim3 grid(g.tile0[g.n], (m + BM - 1) / BM);
  hipLaunchKernelGGL((q4_0_gemm_kernel<BM, BN, MULTI, EPI>), grid, dim3(kThreads), lds, stream, g,
                     cols, x, m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q4_0_gemm(Q40Group g, int cols, const uint16_t *x, int m,
                            hipStream_t stream) {
  // kernels specialised for one matrix and for a plain product
  bool epi = g.gelu != 0;
  for (int k = 0; k < g.n; ++k) epi = epi || g.bias[k] != nullptr;
  if (g.n > 1)
    return epi ? launch_tile<QD_GEMM_BM, QD_GEMM_BN, true, true>(g, cols, x, m, stream)
               : launch_tile<QD_GEMM_BM, QD_GEMM_BN, true, false>(g, cols, x, m, stream);
  return epi ? launch_tile<QD_GEMM_BM, QD_GEMM_BN, false, true>(g, cols, x, m, stream)
             : launch_tile<QD_GEMM_BM, QD_GEMM_BN, false, false>(g, cols, x, m, stream);
}

}  // namespace qd
