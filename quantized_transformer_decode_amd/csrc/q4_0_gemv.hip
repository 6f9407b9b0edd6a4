// q4_0_gemv.hip -- ggml Q4_0 dequant GEMV for gfx950, M <= 16 token rows, f32.
//
// y[t, n] = sum_b d[n,b] * (sum_j q[n,b,j] * x[t,32b+j] - 8 * X[t,b])
// with X[t,b] the sum of x over block b: the "-8" of w = d*(q-8)
// (fuel-transformers 0.19.1, lazy_quantized_whisper.rs -- module
// documentation / quantize_in_out_to_q4_0 for the block format, q_linear for
// the matmul) is folded into one multiply-add per block.  fp32 throughout.
//
// Layout on the chip: a wave covers 8R weight rows; the 8 lanes of a row take
// the blocks b = 8s + lane%8 of step s, so a load instruction reads 8 rows x
// 144 contiguous bytes, and each lane holds R rows whose blocks share its
// reads of x.  A block sits at byte 18*flat (flat = n*bpr + b);
// each lane reads the 4-byte-aligned 20-byte window holding it (starting 2
// bytes early for odd flat -- an even block is never the stream's last, the
// block count per row being a multiple of 8) and realigns the nibbles with
// v_alignbyte_b32.  Loads are unconditional (clamped rows), double-buffered
// in register groups of U steps.  x and the block sums X sit in LDS (fp32);
// up to MT tokens share one pass over the weights.  Small matrices split the
// steps of a row over KS waves of a workgroup (partial sums through LDS).
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kQW = 8;                 // waves per workgroup
constexpr int kQThreads = kQW * kWave;
constexpr int kQMaxSplit = kQW < 8 ? kQW : 8;  // waves one row's steps are split over
constexpr int kQU = 1;                 // steps per register group (2 and 4 measured slower)
constexpr int kQLdsBudget = 64 * 1024;
// x in LDS: each 32-element block padded to 36 floats, so the eight blocks
// one read instruction covers (lanes 8r + j, block j) start in different
// banks (unpadded, blocks 128 bytes apart met four to a bank group: the
// Whisper-base FFN pair at batch 4 10.3 -> 8.7 us)
constexpr int kXBlk = 36;

template <int R>
struct QGroup {
  uint32_t w[kQU][R][5];  // the block windows
  uint32_t odd[kQU][R];   // flat index parities
};

struct QShape {
  int bpr;
  int rg0, stride;      // the wave's first row group and the stride
  int sa, sb;           // the wave's step range
};

// One matrix of a launch, resolved from a row-group index: the row groups of
// the launch's matrices are numbered back to back (matrix k owns
// [tile0[k], tile0[k+1])).
struct QItem {
  const QD_GLOBAL uint8_t *w;
  QD_GLOBAL float *y;
  const float *bias;    // f32 [rows] or null
  int rows;
  int trow;             // first row of the row group in its matrix
};

// Every field of the group descriptor, loaded at the kernel's start: the
// compiler would otherwise load some of them only inside the first branch,
// after the first ones had arrived -- a dependent round trip before the
// first weight load.
__device__ __forceinline__ void q_args_now(const Q40Group &g) {
#pragma unroll
  for (int i = 0; i < kMaxGroup; ++i)
    __asm__ volatile("" ::"s"(g.w[i]), "s"(g.y[i]), "s"(g.bias[i]), "s"(g.rows[i]),
                     "s"(g.tile0[i]));
  __asm__ volatile("" ::"s"(g.tile0[kMaxGroup]), "s"(g.n), "s"(g.gelu), "s"(g.grid),
                   "s"(g.ntiles));
}

// Matrix k's fields by selects over constant indices (indexing the
// kernel-argument arrays with k would be a dependent scalar load).
template <int R>
__device__ __forceinline__ QItem q_item(const Q40Group &grp, int rg) {
  const uint8_t *w = grp.w[0];
  float *y = grp.y[0];
  const float *bias = grp.bias[0];
  int rows = grp.rows[0], t0 = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) {
    const bool in = i < grp.n && rg >= grp.tile0[i];
    w = in ? grp.w[i] : w;
    y = in ? grp.y[i] : y;
    bias = in ? grp.bias[i] : bias;
    rows = in ? grp.rows[i] : rows;
    t0 = in ? grp.tile0[i] : t0;
  }
  QItem it;
  it.w = gp(w);
  it.y = gp(y);
  it.bias = bias;
  it.rows = rows;
  it.trow = (rg - t0) * 8 * R;
  return it;
}

struct QCursor {
  int j, s;             // j-th row group of the wave, step s
};

__device__ __forceinline__ void qc_next(QCursor &c, const QShape &S, int &left) {
  const int adv = left > 1;
  left = adv ? left - 1 : 0;
  const int s = c.s + adv;
  const int wrap = s == S.sb;
  c.s = wrap ? S.sa : s;
  c.j += wrap;
}

// Row r of a lane's R rows in row group g: 8R*g + 8r + lane/8.
template <int R>
__device__ __forceinline__ void qg_issue(QGroup<R> &G, QCursor &c, const QShape &S,
                                         const Q40Group &grp, int lane, int &left) {
#pragma unroll
  for (int u = 0; u < kQU; ++u) {
    const QItem it = q_item<R>(grp, S.rg0 + c.j * S.stride);
    const int base = it.trow + (lane >> 3);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = min(base + 8 * r, it.rows - 1);
      const size_t flat = (size_t)n * S.bpr + 8 * c.s + (lane & 7);
      const uint32_t odd = (uint32_t)(flat & 1);
      const QD_GLOBAL uint32_t *p =
          (const QD_GLOBAL uint32_t *)(it.w + 18 * flat - 2 * odd);
      const u32x4 v = __builtin_nontemporal_load((const QD_GLOBAL u32x4 *)p);
      G.w[u][r][0] = v.x;
      G.w[u][r][1] = v.y;
      G.w[u][r][2] = v.z;
      G.w[u][r][3] = v.w;
      G.w[u][r][4] = __builtin_nontemporal_load(p + 4);
      G.odd[u][r] = odd;
    }
    qc_next(c, S, left);
  }
}

// sum_j q_j x_j over a block for one token and R rows (x read once): nibble
// dword k holds elements 4k..4k+3 (low nibbles) and 16+4k..16+4k+3 (high).
template <int R>
__device__ __forceinline__ void block_dot(const uint32_t (&nib)[R][4], const float *xb,
                                          float (&s)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 a = *(const float4 *)(xb + 4 * k);
    const float4 b = *(const float4 *)(xb + 16 + 4 * k);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t lo = nib[r][k] & 0x0f0f0f0fu, hi = (nib[r][k] >> 4) & 0x0f0f0f0fu;
      s[r] = fmaf(ubyte<0>(lo), a.x, s[r]);
      s[r] = fmaf(ubyte<1>(lo), a.y, s[r]);
      s[r] = fmaf(ubyte<2>(lo), a.z, s[r]);
      s[r] = fmaf(ubyte<3>(lo), a.w, s[r]);
      s[r] = fmaf(ubyte<0>(hi), b.x, s[r]);
      s[r] = fmaf(ubyte<1>(hi), b.y, s[r]);
      s[r] = fmaf(ubyte<2>(hi), b.z, s[r]);
      s[r] = fmaf(ubyte<3>(hi), b.w, s[r]);
    }
  }
}

// Items past the end of the walk are computed with d = 0.
template <int MT, int R, bool STORE, bool EPI>
__device__ __forceinline__ void qg_compute(const QGroup<R> &G, float (&acc)[MT][R], QCursor &c,
                                           const QShape &S, const Q40Group &grp, int &left,
                                           int lane, const float *xs, const float *xsum,
                                           int cols, int t0, int m) {
#pragma unroll
  for (int u = 0; u < kQU; ++u) {
    const int valid = left > 0;  // wave-uniform
    uint32_t nib[R][4];
    float d[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool odd = G.odd[u][r];
      const uint32_t dbits = odd ? (G.w[u][r][0] >> 16) : (G.w[u][r][0] & 0xffffu);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        nib[r][k] = odd ? G.w[u][r][k + 1]
                        : __builtin_amdgcn_alignbyte(G.w[u][r][k + 1], G.w[u][r][k], 2);
      d[r] = valid ? f16_to_f32(dbits) : 0.f;
    }
    const int b = 8 * c.s + (lane & 7);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      float dot[R];
      block_dot<R>(nib, xs + kXBlk * (t * S.bpr + b), dot);
      const float corr = -8.f * xsum[t * S.bpr + b];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[t][r] = fmaf(d[r], dot[r] + corr, acc[t][r]);
    }
    if (STORE && valid && c.s == S.sb - 1) {
      const QItem it = q_item<R>(grp, S.rg0 + c.j * S.stride);
      const int base = it.trow + (lane >> 3);
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float v = group_sum<8>(acc[t][r]);
          const int n = base + 8 * r;
          if ((lane & 7) == 0 && n < it.rows && t0 + t < m)
            it.y[(size_t)(t0 + t) * it.rows + n] =
                EPI ? linear_epilogue(v, it.bias, n, grp.gelu) : v;
          acc[t][r] = 0.f;
        }
    }
    left -= valid;
    const int s = c.s + valid;
    const int wrap = s == S.sb;
    c.s = wrap ? S.sa : s;
    c.j += wrap;
  }
}

template <int MT, int R, int KS, bool EPI>
__global__ __launch_bounds__(kQThreads) void q4_0_gemv_kernel(
    const Q40Group grp, int cols, const float *__restrict__ x_, int t0, int m) {
  static_assert(KS >= 1 && KS <= kQW, "a row's split needs one wave per part");
  q_args_now(grp);
  __asm__ volatile("" ::"s"(x_), "s"(cols), "s"(t0), "s"(m));
  constexpr int SLOTS = kQW / KS;
  __shared__ float red[KS > 1 ? kQW * MT * R * 8 : 1];
  extern __shared__ __attribute__((aligned(16))) float qsh[];
  float *xs = qsh;                    // [MT][bpr] blocks of kXBlk floats
  const int bpr = cols >> 5;
  float *xsum = qsh + MT * bpr * kXBlk;  // [MT][bpr]
  const QD_GLOBAL float *x = gp(x_);
  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);
  const int slot = wave / KS, split = wave % KS;
  const int steps = bpr >> 3;
  QShape S;
  S.bpr = bpr;
  S.sa = uni(steps * split / KS);
  S.sb = uni(steps * (split + 1) / KS);
  S.rg0 = blockIdx.x * SLOTS + slot;
  S.stride = grp.grid * SLOTS;  // the grid size as an argument: gridDim is one more load
  const int ngroups = grp.ntiles;
  int mine = 0;
  if (S.rg0 < ngroups) mine = KS == 1 ? (ngroups - 1 - S.rg0) / S.stride + 1 : 1;
  const int n = uni(mine * (S.sb - S.sa));

  QCursor ci, cc;
  ci.j = cc.j = 0;
  ci.s = cc.s = S.sa;
  int li = n, lc = n;
  QGroup<R> A, B;
  // x staging: thread i copies block i of x (8 x 16 bytes) and its sum, and
  // blocks i + kQThreads, ... after it when there are more blocks than
  // threads.  The first register group of weights is issued between the
  // first x loads and their use, so both are in flight.
  // Block b of the pass (token t0 + b / bpr, block b % bpr of its row) sits
  // at x + t0 * cols + 32 b, the rows being contiguous; blocks of tokens past
  // m (b >= nlive) read the last live block and are staged as zeros.  (No
  // division by the run-time bpr: some forty instructions in front of the
  // first load.)
  const int nblk = MT * bpr;
  const int nlive = min(MT, m - t0) * bpr;
  const QD_GLOBAL float *xt = x + (size_t)t0 * cols;
  const int bi = min((int)threadIdx.x, nblk - 1);
  const QD_GLOBAL floatx4 *xp = (const QD_GLOBAL floatx4 *)(xt + 32 * min(bi, nlive - 1));
  floatx4 xv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) xv[k] = xp[k];
  auto stage = [&]() {
    if ((int)threadIdx.x < nblk) {
      const bool live = bi < nlive;
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const floatx4 v = live ? xv[k] : floatx4{0.f, 0.f, 0.f, 0.f};
        sum += (v[0] + v[1]) + (v[2] + v[3]);
        *(floatx4 *)(xs + kXBlk * bi + 4 * k) = v;
      }
      xsum[bi] = sum;
    }
    for (int b = threadIdx.x + kQThreads; b < nblk; b += kQThreads) {
      const bool live = b < nlive;
      const QD_GLOBAL floatx4 *p = (const QD_GLOBAL floatx4 *)(xt + 32 * min(b, nlive - 1));
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const floatx4 v = live ? p[k] : floatx4{0.f, 0.f, 0.f, 0.f};
        sum += (v[0] + v[1]) + (v[2] + v[3]);
        *(floatx4 *)(xs + kXBlk * b + 4 * k) = v;
      }
      xsum[b] = sum;
    }
  };
  // the staging in both branches: after a join of paths with different
  // numbers of loads in flight the memory waits would be counted for the
  // path with fewer, and the x stores would wait for the weights too
  if (n > 0) {
    qg_issue<R>(A, ci, S, grp, lane, li);
    stage();
  } else {
    stage();
  }
  // LDS writes done, then the barrier (the weight loads stay in flight)
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  float acc[MT][R];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[t][r] = 0.f;
  if (n > 0) {
    // Loads are never conditional; the branches only choose whether another
    // register group is issued before the current one is consumed.
    for (;;) {
      if (lc <= kQU) {
        qg_compute<MT, R, KS == 1, EPI>(A, acc, cc, S, grp, lc, lane, xs, xsum, cols, t0, m);
        break;
      }
      qg_issue<R>(B, ci, S, grp, lane, li);
      qg_compute<MT, R, KS == 1, EPI>(A, acc, cc, S, grp, lc, lane, xs, xsum, cols, t0, m);
      if (lc <= kQU) {
        qg_compute<MT, R, KS == 1, EPI>(B, acc, cc, S, grp, lc, lane, xs, xsum, cols, t0, m);
        break;
      }
      qg_issue<R>(A, ci, S, grp, lane, li);
      qg_compute<MT, R, KS == 1, EPI>(B, acc, cc, S, grp, lc, lane, xs, xsum, cols, t0, m);
    }
  }
  if constexpr (KS > 1) {
    // red[wave][t][row of the group]: the 8-lane sums, written by lane%8 == 0
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = group_sum<8>(acc[t][r]);
        if ((lane & 7) == 0) red[(wave * MT + t) * 8 * R + 8 * r + (lane >> 3)] = v;
      }
    __syncthreads();
    // one thread per (slot, token, row of the group)
    for (int i = threadIdx.x; i < SLOTS * MT * 8 * R; i += kQThreads) {
      const int sl = i / (MT * 8 * R), rem = i - sl * (MT * 8 * R);
      const int t = rem / (8 * R), rr = rem - t * (8 * R);
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < KS; ++k) sum += red[((sl * KS + k) * MT + t) * 8 * R + rr];
      const int rg = blockIdx.x * SLOTS + sl;
      if (rg >= ngroups) continue;
      const QItem it = q_item<R>(grp, rg);
      const int nn = it.trow + rr;
      if (nn < it.rows && t0 + t < m)
        it.y[(size_t)(t0 + t) * it.rows + nn] =
            EPI ? linear_epilogue(sum, it.bias, nn, grp.gelu) : sum;
    }
  }
}

template <int MT, int R, int KS, bool EPI>
hipError_t launch_q_ks(const Q40Group &g, int cols, const float *x, int t0, int m, int grid,
                       hipStream_t stream) {
  const size_t lds = (size_t)MT * (cols / 32) * kXBlk * 4 + (size_t)MT * (cols / 32) * 4;
  if (lds > 48 * 1024) {  // above the default dynamic-LDS limit: raise it once
    static bool raised = false;
    if (!raised) {
      hipError_t e = hipFuncSetAttribute((const void *)q4_0_gemv_kernel<MT, R, KS, EPI>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         kQLdsBudget + 4096);
      if (e != hipSuccess) return e;
      raised = true;
    }
  }
  Q40Group ga = g;
  ga.grid = grid;
  ga.ntiles = g.tile0[g.n];
  hipLaunchKernelGGL((q4_0_gemv_kernel<MT, R, KS, EPI>), dim3(grid), dim3(kQThreads), lds, stream,
                     ga, cols, x, t0, m);
  return hipGetLastError();
}

// KS: split a row's steps over up to kQMaxSplit waves until the launch gives about
// kQTargetWaves waves (each wave keeping at least one register group);
// KS = 1 walks row groups grid-stride with kQStreamWgsPerCu workgroups per CU.
constexpr int kQTargetWaves = 4096;
constexpr int kQStreamWgsPerCu = 2;

template <int MT, bool EPI>
hipError_t launch_q_mt(Q40Group g, int cols, const float *x, int t0, int m,
                       hipStream_t stream) {
  constexpr int R = 1;  // rows per lane
  g.tile0[0] = 0;
  for (int k = 0; k < g.n; ++k) g.tile0[k + 1] = g.tile0[k] + (g.rows[k] + 8 * R - 1) / (8 * R);
  for (int k = g.n; k < kMaxGroup; ++k) g.tile0[k + 1] = g.tile0[g.n];
  const int steps = cols / 256;
  const long ngroups = g.tile0[g.n];
  int ks = 1;
  while (ks < kQMaxSplit && ngroups * ks < kQTargetWaves && steps / (2 * ks) >= kQU) ks *= 2;
  if (ks == 1) {
    int cus = device_cus();
    if (cus < 1) cus = 256;
    long grid = (ngroups + kQW - 1) / kQW;
    if (grid > (long)kQStreamWgsPerCu * cus) grid = (long)kQStreamWgsPerCu * cus;
    return launch_q_ks<MT, R, 1, EPI>(g, cols, x, t0, m, (int)grid, stream);
  }
  const int grid = (int)((ngroups * ks + kQW - 1) / kQW);
  if constexpr (kQMaxSplit >= 2)
    if (ks == 2) return launch_q_ks<MT, R, 2, EPI>(g, cols, x, t0, m, grid, stream);
  if constexpr (kQMaxSplit >= 4)
    if (ks == 4) return launch_q_ks<MT, R, 4, EPI>(g, cols, x, t0, m, grid, stream);
  if constexpr (kQMaxSplit >= 8)
    if (ks == 8) return launch_q_ks<MT, R, 8, EPI>(g, cols, x, t0, m, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_q4_0_gemv(Q40Group g, int cols, const float *x, int m,
                            hipStream_t stream) {
  // tokens per pass limited by the LDS copy of x (fp32 plus block sums)
  const int cap = kQLdsBudget / ((cols / 32) * kXBlk * 4 + cols / 8);
  // kernels specialised for a plain product (no bias, no GELU)
  bool epi = g.gelu != 0;
  for (int k = 0; k < g.n; ++k) epi = epi || g.bias[k] != nullptr;
  int t0 = 0;
  while (t0 < m) {
    const int left = m - t0;
    const int lim = left < cap ? left : cap;
    hipError_t e;
    int mt;
    if (lim >= 4) {
      mt = 4;
      e = epi ? launch_q_mt<4, true>(g, cols, x, t0, m, stream)
              : launch_q_mt<4, false>(g, cols, x, t0, m, stream);
    } else if (lim >= 2) {
      mt = 2;
      e = epi ? launch_q_mt<2, true>(g, cols, x, t0, m, stream)
              : launch_q_mt<2, false>(g, cols, x, t0, m, stream);
    } else {
      mt = 1;
      e = epi ? launch_q_mt<1, true>(g, cols, x, t0, m, stream)
              : launch_q_mt<1, false>(g, cols, x, t0, m, stream);
    }
    if (e != hipSuccess) return e;
    t0 += mt;
  }
  return hipSuccess;
}

}  // namespace qd
