// q4_0_gemm.hip -- Q4_0 prefill GEMM on the gfx950 matrix cores.
//
// y[t, n] = sum_b d[n,b] * P[t,n,b],  P[t,n,b] = sum_j (q[n,b,j]-8) x[t,32b+j]
// (fuel-transformers 0.19.1, lazy_quantized_whisper.rs -- encoder_layer /
// q_linear run every projection over all encoder frames).  The integer codes
// (q - 8) in [-8, 7] are exact in BF16, so each 16x16x32 BF16 MFMA computes
// one block's partial product P exactly up to fp32 accumulation; the f16
// delta is applied to P in fp32 (rounding d*(q-8) to BF16 instead would cost
// up to 2^-9 relative error per weight).  One fp32 multiply-add per output
// per block matches the MFMA's own rate; the VALU does it for block b-1
// while the matrix core runs block b.  (Splitting each weight into two exact
// BF16 halves instead doubles the MFMAs and the LDS reads per output, and
// measured slower.)
//
// Up to four products that share x go in one launch (the q/k/v of a layer):
// their column tiles are numbered back to back and each workgroup looks up
// its matrix.  The q_linear epilogue (f32 bias, gelu_tanh for fc1) is
// applied at the store.
//
// Tiling.  A workgroup owns a (32 x WAVES) frames x 64 weight rows output
// tile; wave w owns frames 32w..32w+31 and all 64 rows (2 x 4 MFMA tiles).
// The waves split the frames only, so each wave's x tile is its own: it is
// loaded in whole cache lines and re-read from a wave-private LDS tile in
// fragment order.  The 64 rows' codes are shared: each stage (128
// columns of K = four Q4_0 blocks) the workgroup converts the raw blocks
// once into exact BF16 codes in LDS ([64][128 + 8], the padding spreading a
// fragment read's 16 rows over all banks) with the deltas in fp32
// ([64][4]), and every wave reads its B fragments there.
//
// Launches with many output tiles (at least 7/4 of 128 x 128 per CU: fc1 of
// a Whisper-large layer at 1500 frames) run a second kernel with 128 x 128
// workgroup tiles and 64 x 64 wave tiles (below).
//
// Launches with fewer output tiles than two per CU (the 1280-row matrices
// of a Whisper-large layer: 240 tiles at 1500 frames) run eight waves per
// workgroup instead: two K parts of four waves, each with its own codes
// buffers, the second part's partial tile added to the first's through LDS
// at the end -- two waves per SIMD instead of one (1280 x 1280: 18.0 ->
// 16.7 us, 1280 x 5120: 56.0 -> 49.0 us).
//
// Pipeline, one barrier per stage.  After the barrier of stage s, a wave
// issues the loads of its x tile of stage s+1 and of the raw blocks of stage
// s+2 (two register sets of these; the loop is unrolled twice so that no set
// is copied), computes stage s from its x tile in LDS and codes buffer s%2
// while converting the raw blocks of stage s+1 into the other buffer (which
// the barrier has just freed: every wave is past stage s-1), and finally
// stores the x tile of stage s+1 over its own.
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int BN = 64;                 // weight rows per workgroup tile
constexpr int BK = 128;                // K columns per stage
constexpr int NB = BK / 32;            // Q4_0 blocks per stage
constexpr int LDB = BK + 8;            // codes row stride in BF16 (272 bytes)
constexpr int TM = 2, TN = 4;          // 16 x 16 MFMA tiles per wave
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

// (q - 8) of four nibbles (one per byte of `n`, bytes in element order) as
// four BF16 in two dwords.  Byte k is placed in the mantissa of 2^23
// (v_perm_b32: bits 0x4b0000qq = 2^23 + q exactly), 2^23 + 8 is subtracted
// exactly, and the small integer converts exactly to BF16.
__device__ __forceinline__ u32x2v codes4_bf16(uint32_t n) {
  floatx4 f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    f[k] = __builtin_bit_cast(float, __builtin_amdgcn_perm(0x4b000000u, n, 0x070c0c00u | k)) -
           8388616.0f;
  return __builtin_bit_cast(u32x2v, __builtin_convertvector(f, bf16x4));
}

// This wave's LDS writes complete, then a workgroup barrier.  No release
// fence: a fence would also wait for the global loads still in flight.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One stage of this wave's 32 frames in flight: load j brings frames
// 4j..4j+3, 256 bytes each (16 lanes per frame).
struct XRegs {
  u32x4 a[8];
};
// The 20-byte window around the Q4_0 block this thread converts.
constexpr int kWaves = 4;  // waves per K part

struct RawRegs {
  u32x4 w4;
  uint32_t w1;
};

template <int WAVES, int KS, bool MULTI, bool EPI>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void q4_0_gemm_kernel(
    const Q40Group grp, int cols, const uint16_t *__restrict__ x, int m) {
  constexpr int FW = WAVES / KS;          // waves per K part (each 32 frames)
  constexpr int PTHREADS = FW * 64;       // threads per K part
  constexpr int BM = FW * 32;
  constexpr int H = PTHREADS / (BN * NB);  // threads per block of a stage: 1 or 2
  static_assert(H == 1 || H == 2, "one block or half a block per thread");
  static_assert(KS == 1 || KS == 2, "K in one or two parts");
  __shared__ __attribute__((aligned(16))) uint16_t codes_all[KS][2][BN * LDB];
  __shared__ __attribute__((aligned(16))) float deltas_all[KS][2][BN * NB];
  // each wave's x tile of the current stage: 32 frames x 16 chunks of 8
  // BF16, chunk c of frame r stored at position c ^ (r % 16)
  __shared__ __attribute__((aligned(16))) u32x4 xs[WAVES][32 * 16];

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
  const uint8_t *w = grp.w[k];
  const int rows = grp.rows[k];
  QD_GLOBAL float *y = gp(grp.y[k]);
  const float *bias = grp.bias[k];
  const int lane = threadIdx.x & 63;
  const int wave = uni((int)threadIdx.x >> 6);
  // K part of this wave, and its place among the part's waves
  const int part = KS == 1 ? 0 : uni(wave / FW);
  const int fw = KS == 1 ? wave : uni(wave - part * FW);
  const int tid = (int)threadIdx.x - part * PTHREADS;
  uint16_t(&codes)[2][BN * LDB] = codes_all[part];
  float(&deltas)[2][BN * NB] = deltas_all[part];
  const int m0 = blockIdx.y * BM;
  const int n0 = (bx - grp.tile0[k]) * BN;
  const int nstages = cols / BK / KS;     // stages of this part
  const int sbase = part * nstages;        // its first stage
  const int nb = cols >> 5;  // Q4_0 blocks per weight row (a multiple of 8)
  const int mrem = min(m - m0, BM), rrem = min(rows - n0, BN);

  // Buffer descriptors over this tile's frames and weight rows; per-stage
  // offsets go in the scalar offset, so the loads take no vector address
  // arithmetic.
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(x + (size_t)m0 * cols), 0, mrem * cols * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(w + (size_t)n0 * nb * 18), 0, rrem * nb * 18, kRsrcWord3);
  const int kc = lane >> 4;  // this lane's chunk (8 K indices) of a block
  // x loads cover whole cache lines: lane l of load j reads chunk l % 16
  // of frame 4j + l / 16 (a fragment-shaped load would touch 16 frames'
  // half lines per instruction, twice the line traffic of the memory
  // pipeline); frames past m read the tile's last frame: they only feed
  // outputs never stored
  int xoff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = min(fw * 32 + 4 * j + (lane >> 4), mrem - 1);
    xoff[j] = r * cols * 2 + (lane & 15) * 16;
  }
  u32x4 *xw = xs[wave];
  // where this lane's loads land in the wave's LDS tile
  int xput[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 4 * j + (lane >> 4);
    xput[j] = r * 16 + ((lane & 15) ^ (r & 15));
  }
  // the block this thread converts: row cr, block cb of each stage
  const int cu = tid / H, ch = tid % H;
  const int cr = cu >> 2, cb = cu & 3;
  const bool cdead = cr >= rrem;  // past the matrix: loads its last row, zeroed
  // 20-byte window holding the block's 18 bytes: 2 bytes early for odd
  // blocks (the block then starts at byte 2 of a dword), on the block for
  // even ones (an even block is never a row's last, so the 2 bytes past it
  // exist); with an even block count per row the parity is cb's
  const int cflat = min(cr, rrem - 1) * nb + cb;
  const int woff = 18 * cflat - 2 * (cb & 1);
  const bool codd = cb & 1;

  auto load_x = [&](XRegs &X, int s) {
    const int so = uni((sbase + s) * BK * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      X.a[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[j], so, 0));
  };
  // the wave's LDS tile is its own: its DS operations run in order, so the
  // tile is rewritten right after the wave's last fragment read of it
  auto put_x = [&](const XRegs &X) {
#pragma unroll
    for (int j = 0; j < 8; ++j) xw[xput[j]] = X.a[j];
  };
  auto load_raw = [&](RawRegs &R, int s) {
    const int so = uni((sbase + s) * NB * 18);
    R.w4 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, woff, so, 0));
    R.w1 = __builtin_amdgcn_raw_buffer_load_b32(wr, woff + 16, so, 0);
  };

  // Quarter i of the conversion of this thread's raw block into buffer buf:
  // dword i of the nibbles (elements 4i..4i+3 in the low nibbles, 16+4i..
  // in the high ones) as exact BF16 codes q - 8; quarter 0 also stores the
  // f16 delta (bytes 0-1 of the block) as fp32.
  auto convert_part = [&](const RawRegs &R, int buf, int i) {
    const uint32_t wv[5] = {R.w4.x, R.w4.y, R.w4.z, R.w4.w, R.w1};
    uint32_t v = codd ? wv[i + 1] : __builtin_amdgcn_alignbyte(wv[i + 1], wv[i], 2);
    v = cdead ? 0x88888888u : v;
    uint16_t *row = &codes[buf][cr * LDB + cb * 32 + 4 * i];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (H == 2 && h != ch) continue;
      const u32x2v cv = codes4_bf16(h ? (v >> 4) & 0x0f0f0f0fu : v & 0x0f0f0f0fu);
      *(u32x2v *)(row + 16 * h) = cv;
    }
    if (i == 0 && ch == 0) {
      const uint32_t dbits = codd ? (wv[0] >> 16) : (wv[0] & 0xffffu);
      deltas[buf][cr * NB + cb] = cdead ? 0.f : f16_to_f32(dbits);
    }
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // the partial products of the last block computed, scaled (by dprev)
  // while the next block's MFMAs run -- across stages too
  floatx4 pprev[TM][TN];
  float dprev[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    dprev[j] = 0.f;
#pragma unroll
    for (int i = 0; i < TM; ++i) pprev[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  auto scale_prev = [&]() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] += dprev[j] * pprev[i][j];
  };

  // One stage from codes buffer buf, interleaved with the conversion of the
  // next stage's raw blocks (R) into the other buffer.  Per block: the B
  // fragments of the next block are read, the block's TM x TN MFMAs issue
  // one by one, and between them the VALU scales the previous block's
  // partial products and converts a quarter of the raw block, so the matrix
  // core and the VALU work at the same time within the wave.
  auto compute = [&](int buf, const RawRegs &R) {
    const uint16_t *B = codes[buf] + (lane & 15) * LDB + kc * 8;
    // A fragment (i, b): frame 16i + lane % 16, chunk 4b + lane / 16
    auto afrag = [&](int i, int b) {
      return __builtin_bit_cast(bf16x8, xw[(16 * i + (lane & 15)) * 16 + ((4 * b + kc) ^ (lane & 15))]);
    };
    bf16x8 af[2][TM];
    const float *D = deltas[buf] + (lane & 15) * NB;
    floatx4 dv[TN];  // deltas of the stage's blocks, per column tile
    bf16x8 bfr[2][TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      dv[j] = *(const floatx4 *)(D + j * 16 * NB);
      bfr[0][j] = *(const bf16x8 *)(B + j * 16 * LDB);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) af[0][i] = afrag(i, 0);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b + 1 < NB) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[(b + 1) & 1][j] = *(const bf16x8 *)(B + j * 16 * LDB + (b + 1) * 32);
#pragma unroll
        for (int i = 0; i < TM; ++i) af[(b + 1) & 1][i] = afrag(i, b + 1);
      }
      floatx4 p[TM][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          p[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              af[b & 1][i], bfr[b & 1][j],
              floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      scale_prev();
      convert_part(R, buf ^ 1, b);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        dprev[j] = dv[j][b];
#pragma unroll
        for (int i = 0; i < TM; ++i) pprev[i][j] = p[i][j];
      }
    }
    // instruction order: per block, the next block's B reads, then each
    // MFMA followed by a share of the VALU work, then the code stores
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * TN + TM, 0);  // DS read
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b > 0) __builtin_amdgcn_sched_group_barrier(0x100, TN + TM, 0);  // DS read
#pragma unroll
      for (int t = 0; t < TM * TN; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 3, 0);  // DS write
    }
  };

  XRegs X;
  RawRegs R0, R1;
  auto step = [&](int s, const RawRegs &Rc, RawRegs &Rl) {
    lds_barrier();  // codes of stage s visible; buffer (s+1)%2 free
    // Past the last stage the loads repeat it and the conversion writes a
    // buffer nobody reads: with no branch, the loop body (two stages; the
    // stage count is even, K being a multiple of 256) is one basic block,
    // so the loads stay ahead of the compute instead of being sunk to their
    // use, and the compiler counts the loads in flight exactly.
    load_x(X, min(s + 1, nstages - 1));
    load_raw(Rl, min(s + 2, nstages - 1));
    __builtin_amdgcn_sched_barrier(0);  // issue them before the compute
    compute(s & 1, Rc);
    put_x(X);  // x of stage s+1, once the wave has read stage s's
  };
  load_x(X, 0);
  load_raw(R0, 0);
  load_raw(R1, min(1, nstages - 1));
#pragma unroll
  for (int i = 0; i < 4; ++i) convert_part(R0, 0, i);
  put_x(X);
  int s = 0;
  for (; s + 1 < nstages; s += 2) {
    step(s, R1, R0);
    step(s + 1, R0, R1);
  }
  if (s < nstages) step(s, R1, R0);  // an odd stage count (K in two parts)
  scale_prev();
  if constexpr (KS == 2) {
    // part 1 hands its partial tile to part 0 through LDS (over the codes
    // buffers, free once every wave is past its last stage)
    float *red = reinterpret_cast<float *>(&codes_all[0][0][0]);
    static_assert(sizeof(codes_all) >= FW * TM * TN * 4 * 64 * sizeof(float), "LDS for the partial tiles");
    __syncthreads();
    if (part == 1) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          *(floatx4 *)(red + (((fw * TM + i) * TN + j) * 64 + lane) * 4) = acc[i][j];
    }
    __syncthreads();
    if (part == 1) return;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] += *(const floatx4 *)(red + (((fw * TM + i) * TN + j) * 64 + lane) * 4);
  }

  float bj[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + j * 16 + (lane & 15);
    bj[j] = (EPI && bias && n < rows) ? ((const QD_GLOBAL float *)bias)[n] : 0.f;
  }
  // C layout of a 16x16 f32 MFMA tile: lane holds rows 4*(lane/16)+v of
  // column lane%16.
  auto store = [&](auto act) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + j * 16 + (lane & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = m0 + fw * 32 + i * 16 + (lane >> 4) * 4 + v;
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

// ---- wide tiles: 128 frames x 128 weight rows per workgroup ----------------
//
// Launches with many output tiles (fc1 of a Whisper-large layer: 480 wide
// tiles at 1500 frames) run 2 x 2 waves of 64 frames x 64 rows each: every
// B fragment read from LDS feeds four MFMAs and every A fragment four, half
// the LDS and L2 traffic per MFMA of the 32 x 64 wave tiles above, and the x
// tile is shared by the two waves of a frame half.  A stage is two Q4_0
// blocks (64 columns: one cache line of each frame), so that two workgroups
// fit a CU (72 KB of LDS each, two waves per SIMD).  Each thread converts
// one raw block per stage into the codes buffer; the x tile is
// double-buffered in LDS like the codes.  A block's partial product is
// scaled by its delta four MFMAs after it is issued (a ring of four
// products), which keeps the scaling off the MFMA's result latency without
// a second set of 16 accumulators.  (fc1 at 1500 frames: 49 -> 43 us; the
// 1280-row matrices have only 120 such tiles and keep the kernel above.)
namespace wide {
constexpr int BM = 128, BN = 128;
constexpr int NB = 2;                  // Q4_0 blocks per stage
constexpr int BK = NB * 32;
constexpr int CH = BK / 8;             // 16-byte chunks of a frame per stage
constexpr int LDB = BK + 8;            // codes row stride in BF16 (144 bytes)
constexpr int TM = 4, TN = 4, NT = TM * TN;
constexpr int LAG = 4;
constexpr int kThreads = 256;
constexpr int XL = BM * CH / kThreads;  // x loads per thread and stage

// Chunk c of frame r in the x tile: rows of 128 bytes, two frames per 64
// banks; sixteen consecutive frames at one chunk land in sixteen distinct
// 16-byte bank groups (fragment reads and line-shaped writes alike).
__device__ __forceinline__ int xslot(int r, int c) { return r * CH + (c ^ ((r >> 1) & 7)); }
}  // namespace wide

template <bool MULTI, bool EPI>
__global__ __launch_bounds__(wide::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void q4_0_gemm_wide_kernel(
    const Q40Group grp, int cols, const uint16_t *__restrict__ x, int m) {
  constexpr int BM = wide::BM, BN = wide::BN, NB = wide::NB, BK = wide::BK, CH = wide::CH;
  constexpr int LDB = wide::LDB, TM = wide::TM, TN = wide::TN, NT = wide::NT, LAG = wide::LAG;
  constexpr int XL = wide::XL;
  using wide::xslot;
  __shared__ __attribute__((aligned(16))) uint16_t codes[2][BN * LDB];
  __shared__ __attribute__((aligned(16))) float deltas[2][BN * NB];
  __shared__ __attribute__((aligned(16))) u32x4 xs[2][BM * CH];

  const int bx = blockIdx.x;
  int k = 0;
  if constexpr (MULTI) {
#pragma unroll
    for (int i = 1; i < kMaxGroup; ++i)
      if (i < grp.n && bx >= grp.tile0[i]) k = i;
    k = uni(k);
  }
  const uint8_t *w = grp.w[k];
  const int rows = grp.rows[k];
  QD_GLOBAL float *y = gp(grp.y[k]);
  const float *bias = grp.bias[k];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // this wave's frame and row halves
  const int m0 = blockIdx.y * BM;
  const int n0 = (bx - grp.tile0[k]) * BN;
  const int nstages = cols / BK;
  const int nb = cols >> 5;
  const int mrem = min(m - m0, BM), rrem = min(rows - n0, BN);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(x + (size_t)m0 * cols), 0, mrem * cols * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(w + (size_t)n0 * nb * 18), 0, rrem * nb * 18, kRsrcWord3);
  const int kc = lane >> 4;

  // x: load j brings chunk tid % 8 of frame 32j + tid / 8 (frames past m
  // read the tile's last frame; they only feed outputs never stored)
  int xoff[XL], xput[XL];
#pragma unroll
  for (int j = 0; j < XL; ++j) {
    const int r = 32 * j + (tid >> 3);
    xoff[j] = min(r, mrem - 1) * cols * 2 + (tid & 7) * 16;
    xput[j] = xslot(r, tid & 7);
  }
  // the block this thread converts: row cr, block cb of each stage (the
  // window and parity rules of the kernel above)
  const int cr = tid >> 1, cb = tid & 1;
  const bool cdead = cr >= rrem;
  const int woff = 18 * (min(cr, rrem - 1) * nb + cb) - 2 * cb;
  const bool codd = cb;

  auto load_x = [&](u32x4 (&X)[XL], int s) {
    const int so = uni(s * BK * 2);
#pragma unroll
    for (int j = 0; j < XL; ++j)
      X[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[j], so, 0));
  };
  auto put_x = [&](const u32x4 (&X)[XL], int buf) {
#pragma unroll
    for (int j = 0; j < XL; ++j) xs[buf][xput[j]] = X[j];
  };
  auto load_raw = [&](RawRegs &R, int s) {
    const int so = uni(s * NB * 18);
    R.w4 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, woff, so, 0));
    R.w1 = __builtin_amdgcn_raw_buffer_load_b32(wr, woff + 16, so, 0);
  };
  // quarter i of the raw block: elements 4i..4i+3 and 16+4i..16+4i+3
  auto convert_part = [&](const RawRegs &R, int buf, int i) {
    const uint32_t wv[5] = {R.w4.x, R.w4.y, R.w4.z, R.w4.w, R.w1};
    uint32_t v = codd ? wv[i + 1] : __builtin_amdgcn_alignbyte(wv[i + 1], wv[i], 2);
    v = cdead ? 0x88888888u : v;
    uint16_t *row = &codes[buf][cr * LDB + cb * 32 + 4 * i];
    *(u32x2v *)(row) = codes4_bf16(v & 0x0f0f0f0fu);
    *(u32x2v *)(row + 16) = codes4_bf16((v >> 4) & 0x0f0f0f0fu);
    if (i == 0) {
      const uint32_t dbits = codd ? (wv[0] >> 16) : (wv[0] & 0xffffu);
      deltas[buf][cr * NB + cb] = cdead ? 0.f : f16_to_f32(dbits);
    }
  };

  floatx4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  // products issued and not yet scaled; slot q of a stage's last LAG are
  // tiles NT-LAG+q of its last block, scaled early in the next stage by rd[q]
  floatx4 ring[LAG];
  float rd[LAG];
#pragma unroll
  for (int q = 0; q < LAG; ++q) {
    ring[q] = floatx4{0.f, 0.f, 0.f, 0.f};
    rd[q] = 0.f;
  }

  // One stage from buffers buf, converting the next stage's raw block (R)
  // into the other codes buffer between the MFMAs.  MFMA u of the stage
  // (block u / NT, tile u % NT = (i, j) = (t / TN, t % TN)) is followed by
  // the scaling of product u - LAG.
  auto compute = [&](int buf, const RawRegs &R) {
    const uint16_t *B = codes[buf] + (64 * wn + (lane & 15)) * LDB + kc * 8;
    const u32x4 *XS = xs[buf];
    auto afrag = [&](int i, int b) {
      return __builtin_bit_cast(bf16x8, XS[xslot(64 * wm + 16 * i + (lane & 15), 4 * b + kc)]);
    };
    const float *D = deltas[buf] + (64 * wn + (lane & 15)) * NB;
    float2 dv[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) dv[j] = *(const float2 *)(D + j * 16 * NB);
    bf16x8 af[2][TM], bfr[2][TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[0][j] = *(const bf16x8 *)(B + j * 16 * LDB);
#pragma unroll
    for (int i = 0; i < TM; ++i) af[0][i] = afrag(i, 0);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b + 1 < NB) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[(b + 1) & 1][j] = *(const bf16x8 *)(B + j * 16 * LDB + (b + 1) * 32);
#pragma unroll
        for (int i = 0; i < TM; ++i) af[(b + 1) & 1][i] = afrag(i, b + 1);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int u = b * NT + t, q = u % LAG;
        const floatx4 pn = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            af[b & 1][t / TN], bfr[b & 1][t % TN], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        if (u >= LAG) {
          const int tt = (u - LAG) % NT;
          const float2 d = dv[tt % TN];
          acc[tt] += ((u - LAG) / NT ? d.y : d.x) * ring[q];
        } else {
          acc[NT - LAG + u] += rd[q] * ring[q];
        }
        ring[q] = pn;
      }
      convert_part(R, buf ^ 1, 2 * b);
      convert_part(R, buf ^ 1, 2 * b + 1);
    }
#pragma unroll
    for (int q = 0; q < LAG; ++q) rd[q] = dv[(NT - LAG + q) % TN].y;
    // per block: the next block's fragment reads, each MFMA followed by a
    // share of the VALU work, then the code stores
    __builtin_amdgcn_sched_group_barrier(0x100, TN + TM, 0);  // DS read
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b > 0) __builtin_amdgcn_sched_group_barrier(0x100, TN + TM, 0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 5, 0);  // DS write
    }
  };

  // Stage s: after the barrier, the x loads of stage s+1 and the raw-block
  // loads of stage s+2 are issued, stage s is computed while stage s+1's raw
  // blocks are converted, and stage s+1's x goes to the other x buffer
  // (free: every wave is past stage s-1).  Past the last stage the loads
  // repeat it, so the two-stage loop body has no branch.
  u32x4 X[XL];
  RawRegs R0, R1;
  auto step = [&](int s, const RawRegs &Rc, RawRegs &Rl) {
    lds_barrier();
    load_x(X, min(s + 1, nstages - 1));
    load_raw(Rl, min(s + 2, nstages - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(s & 1, Rc);
    put_x(X, (s + 1) & 1);
  };
  load_x(X, 0);
  load_raw(R0, 0);
  load_raw(R1, min(1, nstages - 1));
#pragma unroll
  for (int i = 0; i < 4; ++i) convert_part(R0, 0, i);
  put_x(X, 0);
  int s = 0;
  for (; s + 1 < nstages; s += 2) {
    step(s, R1, R0);
    step(s + 1, R0, R1);
  }
  if (s < nstages) step(s, R1, R0);
#pragma unroll
  for (int q = 0; q < LAG; ++q) acc[NT - LAG + q] += rd[q] * ring[q];

  float bj[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + 64 * wn + j * 16 + (lane & 15);
    bj[j] = (EPI && bias && n < rows) ? ((const QD_GLOBAL float *)bias)[n] : 0.f;
  }
  auto store = [&](auto act) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = n0 + 64 * wn + (t % TN) * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tt = m0 + 64 * wm + (t / TN) * 16 + (lane >> 4) * 4 + v;
        if (tt < m && n < rows)
          y[(size_t)tt * rows + n] = EPI ? act(acc[t][v] + bj[t % TN]) : acc[t][v];
      }
    }
  };
  if (EPI && grp.gelu)
    store([](float v) { return linear_epilogue(v, nullptr, 0, 1); });
  else
    store([](float v) { return v; });
}

template <int WAVES, int KS, bool MULTI, bool EPI>
hipError_t launch_tile(const Q40Group &g, int cols, const uint16_t *x, int m, dim3 grid,
                       hipStream_t stream) {
  hipLaunchKernelGGL((q4_0_gemm_kernel<WAVES, KS, MULTI, EPI>), grid, dim3(WAVES * 64), 0, stream,
                     g, cols, x, m);
  return hipGetLastError();
}

// Launches with at least 7/4 wide tiles per CU run the wide kernel; the
// others 128 x 64 tiles, with K split in two parts inside each workgroup
// (eight waves: two waves per SIMD instead of one) when there are fewer
// than two tiles per CU, the parts' partial tiles summed in LDS.
template <bool MULTI, bool EPI>
hipError_t launch_tiles(Q40Group g, int cols, const uint16_t *x, int m, hipStream_t stream) {
  int cus = device_cus();
  if (cus < 1) cus = 256;
  long wide_tiles = 0;
  for (int k = 0; k < g.n; ++k) wide_tiles += (g.rows[k] + wide::BN - 1) / wide::BN;
  wide_tiles *= (m + wide::BM - 1) / wide::BM;
  const int bn = 4 * wide_tiles >= 7L * cus ? wide::BN : BN;
  g.tile0[0] = 0;
  for (int k = 0; k < g.n; ++k) g.tile0[k + 1] = g.tile0[k] + (g.rows[k] + bn - 1) / bn;
  for (int k = g.n; k < kMaxGroup; ++k) g.tile0[k + 1] = g.tile0[g.n];
  if (bn == wide::BN) {
    const dim3 grid(g.tile0[g.n], (m + wide::BM - 1) / wide::BM);
    hipLaunchKernelGGL((q4_0_gemm_wide_kernel<MULTI, EPI>), grid, dim3(wide::kThreads), 0, stream,
                       g, cols, x, m);
    return hipGetLastError();
  }
  constexpr int BM = kWaves * 32;
  const dim3 grid(g.tile0[g.n], (m + BM - 1) / BM);
  if ((long)grid.x * grid.y < 2L * cus)
    return launch_tile<2 * kWaves, 2, MULTI, EPI>(g, cols, x, m, grid, stream);
  return launch_tile<kWaves, 1, MULTI, EPI>(g, cols, x, m, grid, stream);
}

}  // namespace

hipError_t launch_q4_0_gemm(Q40Group g, int cols, const uint16_t *x, int m,
                            hipStream_t stream) {
  // kernels specialised for one matrix and for a plain product
  bool epi = g.gelu != 0;
  for (int k = 0; k < g.n; ++k) epi = epi || g.bias[k] != nullptr;
  if (g.n > 1)
    return epi ? launch_tiles<true, true>(g, cols, x, m, stream)
               : launch_tiles<true, false>(g, cols, x, m, stream);
  return epi ? launch_tiles<false, true>(g, cols, x, m, stream)
             : launch_tiles<false, false>(g, cols, x, m, stream);
}

}  // namespace qd
