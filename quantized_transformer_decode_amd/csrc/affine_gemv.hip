// affine_gemv.hip -- affine-INT8 g64 dequant GEMV for gfx950, M <= 16 token rows.
//
// Computes y[t, r] = sum_c (q[r,c] * s[r,c/64] + b[r,c/64]) * x[t,c]
// (turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- embed_row_bytes for the
// dequantisation, Qwen3AsrMetalEngine::gemv for the GEMV), regrouped per
// 64-column group g as
//   y[t, r] = sum_g s[r,g] * (sum_{c in g} q*x) + b[r,g] * (sum_{c in g} x)
// Codes are exact in fp32, BF16 and f16, accumulation is fp32, the output is
// rounded once (nearest even) to the activation type: BF16, or f16 as in the
// page's Metal GEMV.  Also here: the tied-embedding row lookup
// (embed_row_bytes) on the device.
//
// Two kernels: the matrix-core kernel serves every batch size (one MFMA pair
// per group covers all 16 token rows; the VALU only converts codes and
// applies the group's scale and bias); batch 1 on very large matrices
// streams rows through the VALU instead (one wave per row range, lane l
// holding bytes [16l, 16l+16) of each 1 KiB chunk, x in LDS as fp32).
#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

// ---- small batch: matrix cores ----------------------------------------------
//
// A tile y^T[16 tokens][16 rows] = X[16][K] W^T[K][16] on
// v_mfma_f32_16x16x32_bf16: the A operand is x as given (BF16), the B
// operand the u8 codes converted exactly to BF16.  Per 64-column group g:
//   P[t,n] = sum_{k in g} q[n,k] x[t,k]          (two MFMAs)
//   S[t]   = sum_{k in g} x[t,k]                 (two MFMAs against ones)
//   acc[t,n] += s[n,g] P[t,n] + b[n,g] S[t]      (fp32)
// A lane's four C values (tokens 4*(lane/16)+v, weight row lane%16) share
// one scale and one bias.  K order inside a group: lane quarter g4 = lane/16
// holds columns 16*g4..+7 for the first MFMA and 16*g4+8..+15 for the
// second, for x and codes alike, so each lane reads 16 contiguous code bytes
// and 32 contiguous x bytes per group.  Token rows past m read row m-1 and
// their outputs are dropped.
//
// Work split: a "tile" is 16*R weight rows over all of K.  A workgroup of
// kMW waves has kMW/KS slots of KS waves; the waves of a slot take
// contiguous ranges of the groups and their partial tiles are summed in LDS
// (KS > 1, for matrices with few tiles).  With KS = 1 each wave owns whole
// tiles, walks them grid-stride and stores its own outputs; its loads run
// ahead across tile boundaries (double-buffered, U groups per buffer, always
// issued unconditionally -- past the end the last group is loaded again --
// so the compiler waits only for the buffer being consumed).

constexpr int kMW = 8;
constexpr int kMThreads = kMW * kWave;
constexpr int kMaxDparts = 8;  // partial rows a step prologue sums (one per K/V head)

// Activation type of the matrix-core kernel: x and y BF16 (the configs) or
// f16 (the page's Metal GEMV); scales and biases are BF16 in both.
struct ActBf16 {
  typedef bf16x8 vec;
  static constexpr uint32_t kOnes = 0x3F803F80u;  // two 1.0
  static __device__ __forceinline__ vec codes(uint32_t a, uint32_t b) { return codes8_bf16(a, b); }
  static __device__ __forceinline__ floatx4 mfma(vec a, vec b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t store(float v) { return f32_to_bf16(v); }
};
struct ActF16 {
  typedef halfx8 vec;
  static constexpr uint32_t kOnes = 0x3C003C00u;
  static __device__ __forceinline__ vec codes(uint32_t a, uint32_t b) { return codes8_f16(a, b); }
  static __device__ __forceinline__ floatx4 mfma(vec a, vec b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t store(float v) { return f32_to_f16(v); }
};

// Scales and biases: with CH (the group count a multiple of 4) each buffer
// of U = 4 groups also loads, per 16-row block, one 8-byte piece per lane --
// lanes n and 32+n the scales of row n for the buffer's four groups, lanes
// 16+n and 48+n its biases -- and ds_bpermute hands each lane the pair it
// needs; without CH every lane loads its row's scale and bias per group.
template <int R, int U, bool CH, class A>
struct MGroup {
  u32x4 q[U][R];
  typename A::vec xa[U], xb[U];
  uint16_t sc[CH ? 1 : U][R], bi[CH ? 1 : U][R];
  u32x2 sbv[R];
};

// Walk position: item (j, g) = group g of the wave's j-th tile (wave-uniform).
struct MCursor {
  int j, g;
};

struct MShape {
  int cols, groups;
  int ts0, stride; // the wave's first tile and the tile stride
  int ga, gb;      // the wave's group range
};

// One matrix of a launch, resolved from a tile index: the tiles of the
// group's matrices are numbered back to back (matrix k owns tiles
// [tile0[k], tile0[k+1])).
struct MItem {
  const QD_GLOBAL uint8_t *w;
  const QD_GLOBAL uint16_t *sc;  // scales; biases at sc + boff
  QD_GLOBAL uint16_t *y;
  size_t boff;
  int rows;
  int trow;                      // first row of the tile in its matrix
};

// Every field of the group descriptor, loaded at the kernel's start: the
// compiler would otherwise load some of them only inside the first branch,
// after the first ones had arrived -- a dependent round trip before the
// first weight load.
__device__ __forceinline__ void group_args_now(const AffineGroup &g) {
#pragma unroll
  for (int i = 0; i < kMaxGroup; ++i)
    __asm__ volatile("" ::"s"(g.w[i]), "s"(g.y[i]), "s"(g.rows[i]), "s"(g.tile0[i]));
  __asm__ volatile("" ::"s"(g.tile0[kMaxGroup]), "s"(g.n), "s"(g.grid), "s"(g.ntiles),
                   "s"(g.xdiv));
}

// The descriptor fields of matrix k are picked by selects over constant
// indices: indexing the kernel-argument arrays with k would cost one
// dependent scalar-load round trip per lookup before the first weight load.
template <int R>
__device__ __forceinline__ MItem item_of_tile(const AffineGroup &grp, int cols, int groups,
                                              int tile) {
  int rows = grp.rows[0], t0 = 0;
  const uint8_t *w = grp.w[0];
  uint16_t *y = grp.y[0];
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) {
    const bool in = i < grp.n && tile >= grp.tile0[i];
    rows = in ? grp.rows[i] : rows;
    w = in ? grp.w[i] : w;
    y = in ? grp.y[i] : y;
    t0 = in ? grp.tile0[i] : t0;
  }
  MItem it;
  it.rows = rows;
  it.w = gp(w);
  it.sc = (const QD_GLOBAL uint16_t *)(it.w + (size_t)it.rows * cols);
  it.y = gp(y);
  it.boff = (size_t)it.rows * groups;
  it.trow = (tile - t0) * 16 * R;
  return it;
}

// Advance by one item without branches; `left` counts the items still to
// walk (the cursor stays on the last item once it is 0).
__device__ __forceinline__ void mc_next(MCursor &c, const MShape &S, int &left) {
  const int adv = left > 1;
  left = adv ? left - 1 : 0;
  const int g = c.g + adv;
  const int wrap = g == S.gb;
  c.g = wrap ? S.ga : g;
  c.j += wrap;
}

// Addresses are a wave-uniform base (the tile's first row, the group) plus a
// 32-bit per-lane offset, so the loads take the scalar-base form.  Rows past
// the end of the matrix are clamped to its last row.
// ONE: the wave walks a single tile (K split over the waves of a slot), whose
// matrix and row offsets are resolved once, before the first buffer, rather
// than per item (about 40 scalar instructions per item, in front of the
// first weight loads of a launch).
template <int R, int U, bool CH, bool XL, bool ONE, class A>
__device__ __forceinline__ void mg_issue(MGroup<R, U, CH, A> &G, MCursor &c, const MShape &S,
                                         const AffineGroup &grp,
                                         const QD_GLOBAL uint16_t *x, uint32_t xoff,
                                         const uint8_t *xl, uint32_t xloff, int lane,
                                         int &left, const MItem &it0) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (!XL) {  // with XL, mg_compute reads x from LDS
      const QD_GLOBAL uint8_t *xg = (const QD_GLOBAL uint8_t *)(x + 64 * c.g);
      G.xa[u] = __builtin_bit_cast(typename A::vec, *(const QD_GLOBAL u32x4 *)(xg + xoff));
      G.xb[u] = __builtin_bit_cast(typename A::vec, *(const QD_GLOBAL u32x4 *)(xg + xoff + 16));
    }
    const MItem it = ONE ? it0 : item_of_tile<R>(grp, S.cols, S.groups, S.ts0 + c.j * S.stride);
    const int trow = it.trow;
    const int lim = it.rows - 1 - trow;  // last valid row offset inside the tile
    const QD_GLOBAL uint8_t *cb = it.w + (size_t)trow * S.cols + 64 * c.g;
    const QD_GLOBAL uint8_t *sb =
        (const QD_GLOBAL uint8_t *)(it.sc + (size_t)trow * S.groups + c.g);
    const QD_GLOBAL uint8_t *bb = sb + 2 * it.boff;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // codes: adjacent lanes read adjacent 16-byte pieces (row lane/4,
      // quarter lane%4); mg_compute moves them into the MFMA layout
      const uint32_t co = (uint32_t)min(16 * r + (lane >> 2), lim) * (uint32_t)S.cols +
                          16u * (lane & 3);
      G.q[u][r] = __builtin_nontemporal_load((const QD_GLOBAL u32x4 *)(cb + co));
      const uint32_t so = (uint32_t)min(16 * r + (lane & 15), lim) * (uint32_t)(2 * S.groups);
      if constexpr (CH) {
        if (u == 0)  // the buffer's first group starts a 4-group chunk
          G.sbv[r] = *(const QD_GLOBAL u32x2 *)(((lane >> 4) & 1 ? bb : sb) + so);
      } else {
        G.sc[u][r] = *(const QD_GLOBAL uint16_t *)(sb + so);
        G.bi[u][r] = *(const QD_GLOBAL uint16_t *)(bb + so);
      }
    }
    mc_next(c, S, left);
  }
}

// Output of one finished tile (KS = 1): lane holds tokens 4*(lane/16)+v of
// weight row lane%16 of each 16-row block.
template <int R, class A>
__device__ __forceinline__ void mg_store(floatx4 (&acc)[R], const MShape &S,
                                         const AffineGroup &grp, int j, int m, int lane) {
  const MItem it = item_of_tile<R>(grp, S.cols, S.groups, S.ts0 + j * S.stride);
  const int base = it.trow + (lane & 15);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = base + 16 * r;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = 4 * (lane >> 4) + v;
      if (t < m && n < it.rows) it.y[(size_t)t * it.rows + n] = A::store(acc[r][v]);
      acc[r][v] = 0.f;
    }
  }
}

// Items past the end of the walk (padding up to a whole buffer) are
// computed with zero scale and bias.
template <int R, int U, bool CH, bool STORE, bool XL, class A>
__device__ __forceinline__ void mg_compute(const MGroup<R, U, CH, A> &G, floatx4 (&acc)[R],
                                           MCursor &c, const MShape &S, const AffineGroup &grp,
                                           int &left, int m, int lane, typename A::vec ones,
                                           const uint8_t *xl, uint32_t xloff) {
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  const int src4 = (4 * (lane & 15) + (lane >> 4)) * 4;
  const int srcs = (lane & 15) * 4, srcb = srcs + 64;
  uint32_t sp[R], bp[R];  // scale / bias pair of the current two groups (CH)
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int valid = left > 0;  // wave-uniform
    // x from LDS here rather than with the loads: holding every group's x
    // fragments in registers from issue to use cost 64 VGPRs, one workgroup
    // per CU instead of two (151936 x 1024 at M = 4: 3.9 -> 4.4 TB/s)
    typename A::vec xa, xb;
    if constexpr (XL) {
      const uint8_t *xp = xl + xloff + 128 * c.g;
      xa = *(const typename A::vec *)(xp);
      xb = *(const typename A::vec *)(xp + 16);
    } else {
      xa = G.xa[u];
      xb = G.xb[u];
    }
    floatx4 Sx = A::mfma(xa, ones, z);
    Sx = A::mfma(xb, ones, Sx);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // lane 16*g4 + n takes row n's quarter g4 from lane 4*n + g4
      const u32x4 ql = G.q[u][r];
      const u32x4 q = {(uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)ql.x),
                       (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)ql.y),
                       (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)ql.z),
                       (uint32_t)__builtin_amdgcn_ds_bpermute(src4, (int)ql.w)};
      floatx4 P = A::mfma(xa, A::codes(q.x, q.y), z);
      P = A::mfma(xb, A::codes(q.z, q.w), P);
      float s, b;
      if constexpr (CH) {
        if ((u & 1) == 0) {
          const uint32_t d = u < 2 ? G.sbv[r].x : G.sbv[r].y;
          sp[r] = (uint32_t)__builtin_amdgcn_ds_bpermute(srcs, (int)d);
          bp[r] = (uint32_t)__builtin_amdgcn_ds_bpermute(srcb, (int)d);
        }
        s = __uint_as_float(u & 1 ? sp[r] & 0xffff0000u : sp[r] << 16);
        b = __uint_as_float(u & 1 ? bp[r] & 0xffff0000u : bp[r] << 16);
      } else {
        s = bf16_to_f32(G.sc[u][r]);
        b = bf16_to_f32(G.bi[u][r]);
      }
      s = valid ? s : 0.f;
      b = valid ? b : 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[r][v] = fmaf(s, P[v], fmaf(b, Sx[v], acc[r][v]));
    }
    if (STORE && valid && c.g == S.gb - 1) mg_store<R, A>(acc, S, grp, c.j, m, lane);
    left -= valid;
    const int g = c.g + valid;
    const int wrap = g == S.gb;
    c.g = wrap ? S.ga : g;
    c.j += wrap;
  }
}

// x [m][cols] (16-bit values) into LDS, rows padded to 2*cols + 16 bytes (the
// 16 token rows of a fragment read then start in different banks), 8 chunks
// of 16 bytes per thread at a time.  Chunk i sits at byte 16 i in global
// memory (rows are contiguous) and at 16 (i + row) in LDS, with
// row = i / (cols / 8) by a multiply-high (xdiv): a division by a run-time
// value would put some forty instructions per chunk in front of the loads.
// Past the last chunk a thread repeats it (the same bytes to the same
// place), so the stores need no branch.
__device__ __forceinline__ void stage_x(uint8_t *xl, const QD_GLOBAL uint16_t *x, int chunks,
                                        uint32_t xdiv) {
  for (int base = 0; base < chunks; base += 8 * kMThreads) {
    u32x4 v[8];
    int at[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = min(base + k * kMThreads + (int)threadIdx.x, chunks - 1);
      v[k] = *(const QD_GLOBAL u32x4 *)(x + 8 * i);
      at[k] = 16 * (i + (int)__umulhi((uint32_t)i, xdiv));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) *(u32x4 *)(xl + at[k]) = v[k];
  }
}

__device__ __forceinline__ float round_f16(float v) { return f16_to_f32(f32_to_f16(v)); }

__device__ __forceinline__ float half_of(const u32x4 &w, int e) {
  const uint32_t d = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
  return f16_to_f32((d >> (16 * (e & 1))) & 0xffffu);
}

__device__ __forceinline__ u32x4 pack_halves(const float (&v)[8]) {
  u32x4 r;
  r.x = (uint32_t)f32_to_f16(v[0]) | ((uint32_t)f32_to_f16(v[1]) << 16);
  r.y = (uint32_t)f32_to_f16(v[2]) | ((uint32_t)f32_to_f16(v[3]) << 16);
  r.z = (uint32_t)f32_to_f16(v[4]) | ((uint32_t)f32_to_f16(v[5]) << 16);
  r.w = (uint32_t)f32_to_f16(v[6]) | ((uint32_t)f32_to_f16(v[7]) << 16);
  return r;
}

// The transformed input row (m = 1, f16) into LDS, in the layout of the x staging above
// (GemvPrologue): kind 1 the residual add and RMSNorm, kind 2 SiLU-mul.
// cols <= 8192: at most two 8-value chunks per thread.
// The prologue's global inputs, loaded before the first buffer of weights
// is issued: the memory wait for them then leaves the weight loads in
// flight, and the prologue's arithmetic and barriers overlap the weight
// stream.  PRO 1: x, delta (or the first four columns of each partial row)
// and the norm weights; PRO 2: gate (in xv) and up (in dv).
constexpr int kProCpt = 2;  // 8-element chunks per thread (cols <= 8192)
struct ProIn {
  u32x4 xv[kProCpt], dv[kProCpt], wv[kProCpt];
  floatx4 pv[kMaxDparts];
};

template <int PRO>
__device__ __forceinline__ void pro_load(ProIn &in, const QD_GLOBAL uint16_t *x, int cols,
                                         const GemvPrologue &pro) {
  const int chunks = cols >> 3;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < kProCpt; ++k) {
    const int i = min(t + k * kMThreads, chunks - 1);
    in.xv[k] = *(const QD_GLOBAL u32x4 *)(x + 8 * i);
    if constexpr (PRO == 1) {
      in.wv[k] = *(const QD_GLOBAL u32x4 *)(gp(pro.w) + 8 * i);
      if (pro.delta) in.dv[k] = *(const QD_GLOBAL u32x4 *)(gp(pro.delta) + 8 * i);
    } else {
      in.dv[k] = *(const QD_GLOBAL u32x4 *)(gp(pro.up) + 8 * i);
    }
  }
  if constexpr (PRO == 1) {
    if (pro.dparts) {
      const int c4 = min(t, cols / 4 - 1);
#pragma unroll
      for (int j = 0; j < kMaxDparts; ++j)
        in.pv[j] = *(const QD_GLOBAL floatx4 *)(gp(pro.dparts) +
                                                 (size_t)min(j, pro.nparts - 1) * cols + 4 * c4);
    }
  }
}

template <int PRO>
__device__ __forceinline__ void stage_x_pro(uint8_t *xl, int cols, const GemvPrologue &pro,
                                            const ProIn &in) {
  constexpr int CPT = kProCpt;
  const int chunks = cols >> 3;
  const int t = threadIdx.x;
  float a[CPT][8];
  if constexpr (PRO == 1) {
    __shared__ float red[kMW];
    if (pro.dparts) {
      // delta = f16(dparts[0] + dparts[1] + ...), in that order, staged in
      // LDS as f16 (the norm's row overwrites it after the next barrier)
      for (int c4 = t; c4 < cols / 4; c4 += kMThreads) {
        floatx4 v[kMaxDparts];
#pragma unroll
        for (int j = 0; j < kMaxDparts; ++j)
          v[j] = c4 == t ? in.pv[j]
                         : *(const QD_GLOBAL floatx4 *)(gp(pro.dparts) +
                                                        (size_t)min(j, pro.nparts - 1) * cols +
                                                        4 * c4);
        floatx4 sum = v[0];
#pragma unroll
        for (int j = 1; j < kMaxDparts; ++j)
          if (j < pro.nparts) sum += v[j];
        u32x2 h;
        h.x = (uint32_t)f32_to_f16(sum[0]) | ((uint32_t)f32_to_f16(sum[1]) << 16);
        h.y = (uint32_t)f32_to_f16(sum[2]) | ((uint32_t)f32_to_f16(sum[3]) << 16);
        *(u32x2 *)(xl + 8 * c4) = h;
      }
      __syncthreads();
    }
    const bool has_delta = pro.delta || pro.dparts;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int i = t + k * kMThreads;
      if (i < chunks) {
        u32x4 dv = {0u, 0u, 0u, 0u};
        if (pro.dparts)
          dv = *(const u32x4 *)(xl + 16 * i);
        else if (pro.delta)
          dv = in.dv[k];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          a[k][e] = has_delta ? round_f16(half_of(in.xv[k], e) + half_of(dv, e))
                              : half_of(in.xv[k], e);
          ss = fmaf(a[k][e], a[k][e], ss);
        }
        if (has_delta && pro.x_out && blockIdx.x == 0)
          *(QD_GLOBAL u32x4 *)(gp(pro.x_out) + 8 * i) = pack_halves(a[k]);
      }
    }
    ss = wave_sum(ss);
    if ((t & 63) == 0) red[t >> 6] = ss;
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kMW; ++w) tot += red[w];
    const float inv = 1.f / sqrtf(tot / (float)cols + pro.eps);
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int i = t + k * kMThreads;
      if (i < chunks) {
        const uint32_t we[4] = {in.wv[k].x, in.wv[k].y, in.wv[k].z, in.wv[k].w};
        float n[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          n[e] = a[k][e] * inv * bf16_to_f32((we[e >> 1] >> (16 * (e & 1))) & 0xffffu);
        *(u32x4 *)(xl + 16 * i) = pack_halves(n);
      }
    }
    if (pro.advance && blockIdx.x == 0 && t == 0) gp(pro.advance)[0] += 1;
  } else {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int i = t + k * kMThreads;
      if (i < chunks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float g = half_of(in.xv[k], e);
          a[k][e] = g / (1.f + expf(-g)) * half_of(in.dv[k], e);
        }
        *(u32x4 *)(xl + 16 * i) = pack_halves(a[k]);
      }
    }
  }
}

// PRO != 0: a step GEMV (m = 1, f16, XL) reading the row that stage_x_pro
// builds.
template <int R, int U, int KS, bool CH, bool XL, class Act, int PRO>
__global__ __launch_bounds__(kMThreads) void affine_gemv_mfma_kernel(
    const AffineGroup grp, int cols, const uint16_t *__restrict__ x_, int m,
    const GemvPrologue pro) {
  group_args_now(grp);
  constexpr int SLOTS = kMW / KS;
  __shared__ float red[KS > 1 ? kMW * R * kWave * 4 : 1];
  extern __shared__ __attribute__((aligned(16))) uint8_t xsh[];  // x (XL)
  uint8_t *xl = xsh;
  __asm__ volatile("" ::"s"(x_), "s"(cols), "s"(m));
  const int lane = threadIdx.x & 63;
  const int wave = uni(threadIdx.x >> 6);
  const int slot = wave / KS, split = wave % KS;
  MShape S;
  S.cols = cols;
  S.groups = cols >> 6;
  // group ranges in whole buffers of U groups when the scales come in chunks
  const int unit = CH ? U : 1;
  const int units = S.groups / unit;
  S.ga = uni(unit * (units * split / KS));
  S.gb = uni(unit * (units * (split + 1) / KS));
  S.ts0 = blockIdx.x * SLOTS + slot;
  S.stride = grp.grid * SLOTS;  // the grid size as an argument: gridDim is one more load
  const int ntiles = grp.ntiles;
  int tiles_mine = 0;
  if (S.ts0 < ntiles) tiles_mine = KS == 1 ? (ntiles - 1 - S.ts0) / S.stride + 1 : 1;
  const int n = uni(tiles_mine * (S.gb - S.ga));
  const int t = (lane & 15) < m ? (lane & 15) : m - 1;
  const QD_GLOBAL uint16_t *x = gp(x_);
  const uint32_t xoff = 2u * ((uint32_t)t * (uint32_t)cols + 16u * (lane >> 4));  // bytes
  const uint32_t xloff = (uint32_t)t * (2u * cols + 16u) + 32u * (lane >> 4);

  floatx4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = floatx4{0.f, 0.f, 0.f, 0.f};
  const typename Act::vec ones = __builtin_bit_cast(
      typename Act::vec, u32x4{Act::kOnes, Act::kOnes, Act::kOnes, Act::kOnes});
  // the single tile of a split wave (KS > 1; past the last tile the wave
  // has no items and the clamped tile is never read)
  MItem it0 = {};
  if constexpr (KS > 1)
    it0 = item_of_tile<R>(grp, cols, S.groups, min(S.ts0, ntiles - 1));
  MCursor ci, cc;  // issue and compute cursors
  ci.j = cc.j = 0;
  ci.g = cc.g = S.ga;
  int li = n, lc = n;
  MGroup<R, U, CH, Act> A, B;
  // the first buffer's codes and scales are in flight while x is staged;
  // a prologue's inputs are loaded first, so that waiting for them does not
  // wait for the weights
  ProIn pin;
  if constexpr (XL && PRO != 0) {
    pro_load<PRO>(pin, x, cols, pro);
    // the prologue in both branches: after a join of paths with different
    // numbers of loads in flight, the memory waits would be counted for
    // the path with fewer (and wait for the weights here too)
    if (n > 0) {
      mg_issue<R, U, CH, XL, (KS > 1), Act>(A, ci, S, grp, x, xoff, xl, xloff, lane, li, it0);
      stage_x_pro<PRO>(xl, cols, pro, pin);
    } else {
      stage_x_pro<PRO>(xl, cols, pro, pin);
    }
  } else {
    if (n > 0)
      mg_issue<R, U, CH, XL, (KS > 1), Act>(A, ci, S, grp, x, xoff, xl, xloff, lane, li, it0);
    if constexpr (XL) stage_x(xl, x, m * (cols >> 3), grp.xdiv);
  }
  if constexpr (XL) {
    // LDS writes done, then the barrier (global loads stay in flight)
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if (n > 0) {
    // Loads are never conditional (the compiler then waits for exactly the
    // buffer it consumes); the branches only choose whether another buffer
    // is issued before the current one is consumed.
    for (;;) {
      if (lc <= U) {
        mg_compute<R, U, CH, KS == 1, XL, Act>(A, acc, cc, S, grp, lc, m, lane, ones, xl, xloff);
        break;
      }
      mg_issue<R, U, CH, XL, (KS > 1), Act>(B, ci, S, grp, x, xoff, xl, xloff, lane, li, it0);
      mg_compute<R, U, CH, KS == 1, XL, Act>(A, acc, cc, S, grp, lc, m, lane, ones, xl, xloff);
      if (lc <= U) {
        mg_compute<R, U, CH, KS == 1, XL, Act>(B, acc, cc, S, grp, lc, m, lane, ones, xl, xloff);
        break;
      }
      mg_issue<R, U, CH, XL, (KS > 1), Act>(A, ci, S, grp, x, xoff, xl, xloff, lane, li, it0);
      mg_compute<R, U, CH, KS == 1, XL, Act>(B, acc, cc, S, grp, lc, m, lane, ones, xl, xloff);
    }
  }
  if constexpr (KS > 1) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[((wave * R + r) * kWave + lane) * 4 + v] = acc[r][v];
    __syncthreads();
    for (int i = threadIdx.x; i < SLOTS * R * kWave * 4; i += kMThreads) {
      const int sl = i / (R * kWave * 4), rem = i - sl * (R * kWave * 4);
      const int r = rem >> 8, l = (rem >> 2) & 63, v = rem & 3;
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < KS; ++k) sum += red[(((sl * KS + k) * R + r) * kWave + l) * 4 + v];
      const int tile = blockIdx.x * SLOTS + sl;
      if (tile >= ntiles) continue;
      const MItem it = item_of_tile<R>(grp, cols, S.groups, tile);
      const int tt = 4 * (l >> 4) + v;
      const int nn = it.trow + 16 * r + (l & 15);
      if (tt < m && nn < it.rows) it.y[(size_t)tt * it.rows + nn] = Act::store(sum);
    }
  }
}

// Matrix-core kernel shape: 16-row tiles (R = 1); K is split until a launch
// has about 4096 waves; the streaming walk (KS = 1) runs two workgroups per
// CU.
constexpr int kAffineR = 1;
constexpr int kAffineTargetWaves = 4096;
constexpr int kAffineStreamWgsPerCu = 2;

// x goes to LDS when its padded copy fits this budget (two workgroups per
// CU then still fit the 160 KiB of LDS).
constexpr int kXlBudget = 72 * 1024;

template <int KS, bool CH, bool XL, class Act, int PRO>
hipError_t launch_mfma_ks(const AffineGroup &g, int cols, const uint16_t *x, int m, int grid,
                          const GemvPrologue &pro, hipStream_t stream) {
  constexpr int R = kAffineR;
  constexpr int U = CH ? 4 : 2;
  const size_t lds = XL ? (size_t)m * (2 * cols + 16) : 0;
  if (lds > 48 * 1024) {  // above the default dynamic-LDS limit: raise it once
    static bool raised = false;
    if (!raised) {
      hipError_t e = hipFuncSetAttribute(
          (const void *)affine_gemv_mfma_kernel<R, U, KS, CH, XL, Act, PRO>,
          hipFuncAttributeMaxDynamicSharedMemorySize, kXlBudget);
      if (e != hipSuccess) return e;
      raised = true;
    }
  }
  AffineGroup ga = g;
  ga.grid = grid;
  ga.ntiles = g.tile0[g.n];
  const uint64_t per_row = (uint64_t)cols / 8;
  ga.xdiv = (uint32_t)(((1ull << 32) + per_row - 1) / per_row);
  hipLaunchKernelGGL((affine_gemv_mfma_kernel<R, U, KS, CH, XL, Act, PRO>), dim3(grid),
                     dim3(kMThreads), lds, stream, ga, cols, x, m, pro);
  return hipGetLastError();
}

// The streaming walk (KS = 1) stages x: there a workgroup reuses it over
// many tiles.  A split workgroup reads each element of x once anyway, but
// with m > 1 its x fragments held in registers from issue to use cost 150
// VGPRs, one workgroup per CU; staged, they are read at use (107 VGPRs, two
// per CU: the Qwen3-1.7B step at M = 16 1.155 -> 1.120 ms).  At m = 1 the
// staging's extra round trip and barrier cost more than that (1024 x 1024:
// 3.5 -> 4.3 us per launch).  A prologue always stages (the transformed row
// exists only in LDS).
template <int KS, bool CH, class Act, int PRO>
hipError_t launch_mfma_xl(const AffineGroup &g, int cols, const uint16_t *x, int m, int grid,
                          const GemvPrologue &pro, hipStream_t stream) {
  if constexpr (PRO != 0) {
    return launch_mfma_ks<KS, CH, true, Act, PRO>(g, cols, x, m, grid, pro, stream);
  } else {
    if ((KS == 1 || m > 1) && (size_t)m * (2 * cols + 16) <= (size_t)kXlBudget)
      return launch_mfma_ks<KS, CH, true, Act, PRO>(g, cols, x, m, grid, pro, stream);
    return launch_mfma_ks<KS, CH, false, Act, PRO>(g, cols, x, m, grid, pro, stream);
  }
}

template <bool CH, class Act, int PRO>
hipError_t launch_mfma_ch(AffineGroup g, int cols, const uint16_t *x, int m,
                          const GemvPrologue &pro, hipStream_t stream) {
  // KS: split K over up to 8 waves until the launch gives about
  // kTargetWaves waves (each wave keeping at least one buffer of groups);
  // KS = 1 walks tiles grid-stride with kStreamWgsPerCu workgroups per CU.
  constexpr int kTargetWaves = kAffineTargetWaves;
  constexpr int kStreamWgsPerCu = kAffineStreamWgsPerCu;
  constexpr int R = kAffineR;
  g.tile0[0] = 0;
  for (int k = 0; k < g.n; ++k) g.tile0[k + 1] = g.tile0[k] + (g.rows[k] + 16 * R - 1) / (16 * R);
  for (int k = g.n; k < kMaxGroup; ++k) g.tile0[k + 1] = g.tile0[g.n];
  const int units = (cols / 64) / (CH ? 4 : 1);
  const long ntiles = g.tile0[g.n];
  int ks = 1;
  while (ks < 8 && ntiles * ks < kTargetWaves && units / (2 * ks) >= (CH ? 1 : 2)) ks *= 2;
  if (ks == 1) {
    int cus = device_cus();
    if (cus < 1) cus = 256;
    long grid = (ntiles + kMW - 1) / kMW;
    if (grid > (long)kStreamWgsPerCu * cus) grid = (long)kStreamWgsPerCu * cus;
    return launch_mfma_xl<1, CH, Act, PRO>(g, cols, x, m, (int)grid, pro, stream);
  }
  const int grid = (int)((ntiles * ks + kMW - 1) / kMW);
  switch (ks) {
    case 2: return launch_mfma_xl<2, CH, Act, PRO>(g, cols, x, m, grid, pro, stream);
    case 4: return launch_mfma_xl<4, CH, Act, PRO>(g, cols, x, m, grid, pro, stream);
    default: return launch_mfma_xl<8, CH, Act, PRO>(g, cols, x, m, grid, pro, stream);
  }
}

template <class Act, int PRO = 0>
hipError_t launch_mfma(const AffineGroup &g, int cols, const uint16_t *x, int m,
                       const GemvPrologue &pro, hipStream_t stream) {
  if ((cols / 64) % 4 == 0) return launch_mfma_ch<true, Act, PRO>(g, cols, x, m, pro, stream);
  return launch_mfma_ch<false, Act, PRO>(g, cols, x, m, pro, stream);
}

// ---- batch 1: streaming kernel ---------------------------------------------
//
// Each wave owns a contiguous range of rows and walks its items -- (row,
// 1 KiB chunk) pairs, lane l holding bytes [16l, 16l+16) of the chunk -- in
// register groups of kG items, double-buffered: the next group's loads are
// issued (always the same number, so the compiler waits for exactly the
// group being consumed) before the current group is computed.  x sits in LDS
// in the xswz layout, fp32.  Groups of two items with up to four
// workgroups per CU measured fastest on the LM heads (8 items: ~10-30 %
// slower; 8 workgroups per CU: no better).

constexpr int kG = 2;
constexpr int kM1Threads = 512;
constexpr int kM1Cpt = 2;  // 8-element pieces of x per thread (cols <= 8192)
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

template <bool F16>
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
        if (lane == 0) y[row] = F16 ? f32_to_f16(rowsum) : f32_to_bf16(rowsum);
        rowsum = 0.f;
      }
      if (++ch == chunks) {
        ch = 0;
        ++row;
      }
    }
  }
}

// x and y BF16, or f16 with F16.  PRO = 1 (f16 only): the staged row is the
// residual add + RMSNorm of GemvPrologue kind 1 (the decoder step's final
// norm before the tied LM head).
template <bool F16, int PRO>
__global__ __launch_bounds__(kM1Threads) void affine_gemv_m1_kernel(
    const uint8_t *__restrict__ w_, int rows, int cols, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y_, const GemvPrologue pro) {
  extern __shared__ __attribute__((aligned(16))) float xl[];  // chunks*1024, xswz layout
  const int chunks = (cols + 1023) >> 10;
  // x (with PRO 1 also delta and the norm weights) as 16-byte pieces of 8
  // elements, every load issued before any is used, and before the first
  // weights: the staging then costs one memory round trip, under the
  // weight stream
  const int c8 = cols >> 3, t = threadIdx.x;
  u32x4 xv[kM1Cpt], dv[kM1Cpt], wv[kM1Cpt];
#pragma unroll
  for (int k = 0; k < kM1Cpt; ++k) {
    const int i = min(t + k * kM1Threads, c8 - 1);
    xv[k] = *(const QD_GLOBAL u32x4 *)(gp(x) + 8 * i);
    if constexpr (PRO == 1) {
      wv[k] = *(const QD_GLOBAL u32x4 *)(gp(pro.w) + 8 * i);
      if (pro.delta) dv[k] = *(const QD_GLOBAL u32x4 *)(gp(pro.delta) + 8 * i);
    }
  }
  auto put8 = [&](int i, const float (&v)[8]) {
    *(floatx4 *)(xl + xswz(8 * i)) = floatx4{v[0], v[1], v[2], v[3]};
    *(floatx4 *)(xl + xswz(8 * i + 4)) = floatx4{v[4], v[5], v[6], v[7]};
  };
  auto stage = [&]() {
    if constexpr (PRO == 1) {
      __shared__ float red[kM1Waves];
      float a[kM1Cpt][8];
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < kM1Cpt; ++k) {
        const int i = t + k * kM1Threads;
        if (i < c8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            a[k][e] = pro.delta ? round_f16(half_of(xv[k], e) + half_of(dv[k], e))
                                : half_of(xv[k], e);
            ss = fmaf(a[k][e], a[k][e], ss);
          }
          if (pro.delta && pro.x_out && blockIdx.x == 0)
            *(QD_GLOBAL u32x4 *)(gp(pro.x_out) + 8 * i) = pack_halves(a[k]);
        }
      }
      ss = wave_sum(ss);
      if ((t & 63) == 0) red[t >> 6] = ss;
      __syncthreads();
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kM1Waves; ++w) tot += red[w];
      const float inv = 1.f / sqrtf(tot / (float)cols + pro.eps);
#pragma unroll
      for (int k = 0; k < kM1Cpt; ++k) {
        const int i = t + k * kM1Threads;
        if (i < c8) {
          const uint32_t we[4] = {wv[k].x, wv[k].y, wv[k].z, wv[k].w};
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            v[e] = round_f16(a[k][e] * inv * bf16_to_f32((we[e >> 1] >> (16 * (e & 1))) & 0xffffu));
          put8(i, v);
        }
      }
      if (pro.advance && blockIdx.x == 0 && t == 0) gp(pro.advance)[0] += 1;
    } else {
#pragma unroll
      for (int k = 0; k < kM1Cpt; ++k) {
        const int i = t + k * kM1Threads;
        if (i < c8) {
          const uint32_t xe[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t b = (xe[e >> 1] >> (16 * (e & 1))) & 0xffffu;
            v[e] = F16 ? f16_to_f32(b) : bf16_to_f32(b);
          }
          put8(i, v);
        }
      }
    }
  };
  const QD_GLOBAL uint8_t *w = gp(w_);
  QD_GLOBAL uint16_t *y = gp(y_);
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * kM1Waves;
  const int gw = blockIdx.x * kM1Waves + uni(threadIdx.x >> 6);
  const int lo = uni((int)(((int64_t)rows * gw) / nw));
  const int hi = uni((int)(((int64_t)rows * (gw + 1)) / nw));
  const int n = uni((hi - lo) * chunks);
  M1Group A, B;
  // the staging in both branches: after a join of paths with different
  // numbers of loads in flight the memory waits would be counted for the
  // path with fewer, and the staging would wait for the first weights
  if (n > 0) {
    m1_issue(A, w, rows, cols, chunks, lo, n, 0, lane);
    stage();
  } else {
    stage();
  }
  __syncthreads();
  if (n == 0) return;
  float rowsum = 0.f;
  for (int i = 0; i < n; i += 2 * kG) {
    m1_issue(B, w, rows, cols, chunks, lo, n, i + kG < n ? i + kG : i, lane);
    m1_compute<F16>(A, cols, chunks, lo, n, i, lane, xl, y, rowsum);
    if (i + kG >= n) break;
    m1_issue(A, w, rows, cols, chunks, lo, n, i + 2 * kG < n ? i + 2 * kG : i + kG, lane);
    m1_compute<F16>(B, cols, chunks, lo, n, i + kG, lane, xl, y, rowsum);
  }
}

// ---- tied-embedding rows ------------------------------------------------------
//
// out[i, c] = round16(fl32(q[t_i, c] * s + b)) (embed_row_bytes): q*s is
// exact in fp32, so one fused multiply-add gives the page's f32 value; it is
// then rounded to f16 or BF16.  Each thread handles four columns of one
// group; blockIdx.y is the token.
constexpr int kEmbedThreads = 256;

__global__ __launch_bounds__(kEmbedThreads) void affine_embed_rows_kernel(
    const uint8_t *__restrict__ w_, int rows, int cols, const EmbedTokens tk,
    uint16_t *__restrict__ out_, int f16) {
  const int c = (blockIdx.x * kEmbedThreads + threadIdx.x) * 4;
  if (c >= cols) return;
  const int i = blockIdx.y;
  const size_t tok = (size_t)tk.t[i];
  const QD_GLOBAL uint8_t *w = gp(w_);
  const int groups = cols >> 6;
  const uint32_t q = *(const QD_GLOBAL uint32_t *)(w + tok * cols + c);
  const QD_GLOBAL uint16_t *sc = (const QD_GLOBAL uint16_t *)(w + (size_t)rows * cols);
  const size_t gi = tok * groups + (c >> 6);
  const float s = bf16_to_f32(sc[gi]);
  const float b = bf16_to_f32(sc[(size_t)rows * groups + gi]);
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float v = fmaf((float)((q >> (8 * k)) & 0xffu), s, b);
    // Two roundings, as the page has them: the f32 value, then the 16-bit
    // store.  The empty asm makes v opaque: the compiler would otherwise
    // fuse the multiply-add and the f16 conversion into one
    // v_fma_mixlo_f16, which rounds the exact value to f16 once and can
    // differ in the last bit.
    __asm__("" : "+v"(v));
    o[k] = f16 ? f32_to_f16(v) : f32_to_bf16(v);
  }
  *(QD_GLOBAL u32x2 *)(gp(out_) + (size_t)i * cols + c) =
      u32x2{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
}

}  // namespace

hipError_t launch_affine_embed_rows(const uint8_t *w, int rows, int cols, const EmbedTokens &tk,
                                    uint16_t *out, bool f16, hipStream_t stream) {
  dim3 grid((cols / 4 + kEmbedThreads - 1) / kEmbedThreads, tk.n);
  hipLaunchKernelGGL(affine_embed_rows_kernel, grid, dim3(kEmbedThreads), 0, stream, w, rows,
                     cols, tk, out, f16 ? 1 : 0);
  return hipGetLastError();
}

// Batch 1 takes the VALU streaming kernel only for a single very large
// matrix (LM heads, >= 2^27 weights), where its 1 KiB-per-row loads keep the
// most bytes in flight (151936 x 1024: 5.2-5.4 TB/s against ~4.0 for the
// matrix-core kernel); below that the matrix-core kernel's K split gives
// more waves.
static bool use_m1(const AffineGroup &g, int cols, int m) {
  return g.n == 1 && m == 1 && (int64_t)g.rows[0] * cols >= ((int64_t)1 << 27);
}

template <bool F16, int PRO>
static hipError_t launch_m1(const AffineGroup &g, int cols, const uint16_t *x,
                            const GemvPrologue &pro, hipStream_t stream) {
  const uint8_t *w = g.w[0];
  uint16_t *y = g.y[0];
  const int rows = g.rows[0];
  // waves: about two register groups of items each, at most 4 workgroups
  // of 8 waves per CU
  int cus = device_cus();
  if (cus < 1) cus = 256;
  const int64_t items = (int64_t)rows * ((cols + 1023) / 1024);
  int64_t wgs = (items + 2 * kG * kM1Waves - 1) / (2 * kG * kM1Waves);
  if (wgs > 4 * (int64_t)cus) wgs = 4 * (int64_t)cus;
  if (wgs < 1) wgs = 1;
  const size_t lds = (size_t)((cols + 1023) / 1024) * 1024 * 4;
  hipLaunchKernelGGL((affine_gemv_m1_kernel<F16, PRO>), dim3((unsigned)wgs), dim3(kM1Threads),
                     lds, stream, w, rows, cols, x, y, pro);
  return hipGetLastError();
}

hipError_t launch_affine_gemv(AffineGroup g, int cols, const uint16_t *x, int m, bool f16,
                              hipStream_t stream) {
  const GemvPrologue none = {};
  if (use_m1(g, cols, m))
    return f16 ? launch_m1<true, 0>(g, cols, x, none, stream)
               : launch_m1<false, 0>(g, cols, x, none, stream);
  if (f16) return launch_mfma<ActF16>(g, cols, x, m, none, stream);
  return launch_mfma<ActBf16>(g, cols, x, m, none, stream);
}

hipError_t launch_affine_gemv_pro(AffineGroup g, int cols, const uint16_t *x,
                                  const GemvPrologue &pro, hipStream_t stream) {
  if (pro.kind == 1 && pro.dparts && (pro.nparts < 1 || pro.nparts > kMaxDparts))
    return hipErrorInvalidValue;
  if (pro.kind == 1 && !pro.dparts && use_m1(g, cols, 1))
    return launch_m1<true, 1>(g, cols, x, pro, stream);
  if (pro.kind == 1) return launch_mfma<ActF16, 1>(g, cols, x, 1, pro, stream);
  if (pro.kind == 2) return launch_mfma<ActF16, 2>(g, cols, x, 1, pro, stream);
  return launch_mfma<ActF16>(g, cols, x, 1, pro, stream);
}

}  // namespace qd
