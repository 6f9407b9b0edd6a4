// attention.hip -- decode attention over the K/V cache (grouped-query), one
// query row per head, split softmax.
//
// turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::step
// runs encode_attention_decode after the K/V projections have written the
// current position's row into the cache: every query head h attends the rows
// [kv_start, length) of K/V head h / (heads / kv_heads),
//   out[h] = softmax_t(scale * q[h] . k[t]) v[t].
// The cache row of position t holds all K/V heads ([rows][kv_heads][d]).
//
// Split softmax (the page keeps a split-softmax scratch for this): the
// positions are cut into chunks; a workgroup takes one K/V head and one
// chunk, for every query head of the group, so each cached row is read once
// per group.  Inside a wave, d/8 lanes share a row (8 dimensions, 16 bytes
// each) and the wave covers 64 / (d/8) rows per load; every lane keeps an
// online softmax (running max m, sum l, output o) of the rows it has seen,
// merged across lanes with shuffles and across waves in LDS.  A second
// kernel, one workgroup per query head, combines the chunks' (m, l, o):
// M = max m, out = sum o e^(m-M) / sum l e^(m-M); a window that fits one
// chunk is normalised and stored by the first kernel.  Scores, exponentials
// and sums are fp32; the output is rounded once to the 16-bit activation
// type.  (Folding the combine into the first kernel -- the last workgroup
// of a K/V head merging it -- measured slower at every window size: that
// one workgroup's chain of memory round trips costs more than the second
// launch.)  Inside the decoder step, the first kernel also takes over the
// per-head q/k RMSNorm + RoPE and the K/V cache append (QKR).
#include <atomic>

#include "qd_device.h"
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kAttThreads = 256;
constexpr int kAttWaves = kAttThreads / kWave;
constexpr int kAttUnroll = 2;      // row loads in flight per lane (K and V each)
constexpr int kAttTargetWgs = 512; // about two workgroups per CU of a 256-CU device
constexpr int kAttSingleRowsPerWave = 32;  // windows up to 4 * 32 rows: a single chunk

// With a device position the grid (gchunks chunks per K/V head) is sized for
// the whole cache, and the chunk length follows the live window of len rows:
// about 1.5 sqrt(len) rows, at least 32 (and at most gchunks chunks), in
// whole row loads per wave.  Measured in the decoder step, the best length
// grows with the window: 32-row chunks at 128 rows, 64 at 1024, 96 at 4096
// (64, 128 and 256 are slower there).  Every kernel of a call derives it the
// same way.
template <int D>
__device__ __forceinline__ int att_dev_rows_per_wave(int len, int gchunks) {
  constexpr int step = (kWave / (D / 8)) * kAttUnroll;
  int rows = max(32, (int)(1.5f * sqrtf((float)len)));
  rows = max(rows, (len + gchunks - 1) / gchunks);
  const int want = (rows + kAttWaves - 1) / kAttWaves;
  // wave-uniform: kept in a scalar register, so the row loop stays scalar
  return uni(max(step, (want + step - 1) / step * step));
}

template <bool F16>
__device__ __forceinline__ float to_f32(uint32_t bits) {
  return F16 ? f16_to_f32(bits) : bf16_to_f32(bits);
}

template <bool F16>
__device__ __forceinline__ void unpack8(const u32x4 w, float (&f)[8]) {
  const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = to_f32<F16>(e[i] & 0xffffu);
    f[2 * i + 1] = to_f32<F16>(e[i] >> 16);
  }
}

// Merge (m2, l2, o2) into (m, l, o); m = -inf marks an empty state.
template <int G>
__device__ __forceinline__ void merge(float (&m)[G], float (&l)[G], float (&o)[G][8],
                                      const float (&m2)[G], const float (&l2)[G],
                                      const float (&o2)[G][8]) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mm = fmaxf(m[h], m2[h]);
    const float a = m[h] == -INFINITY ? 0.f : __expf(m[h] - mm);
    const float b = m2[h] == -INFINITY ? 0.f : __expf(m2[h] - mm);
    l[h] = l[h] * a + l2[h] * b;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[h][i] = o[h][i] * a + o2[h][i] * b;
    m[h] = mm;
  }
}

template <bool F16>
__device__ __forceinline__ uint16_t store16(float v) {
  return F16 ? f32_to_f16(v) : f32_to_bf16(v);
}

// The d outputs of one query head from its nchunks partials (layout of
// attention_partial_kernel), by one workgroup: S = 256 / d slices of the
// chunks run side by side, thread t taking dimension t % d of slice t / d,
// and merge in LDS.  Chunks are read kCombBatch at a time with independent
// loads, and each batch is folded in against its own maximum, so a head
// costs about nchunks / (S * kCombBatch) memory round trips.
constexpr int kCombBatch = 16;
template <int D, bool F16>
__device__ __forceinline__ void combine_chunks(const QD_GLOBAL float *part, int nchunks,
                                               QD_GLOBAL uint16_t *out) {
  constexpr int S = kAttThreads / D;
  __shared__ float sm[S][D], sl[S][D], so[S][D];
  const int t = threadIdx.x;
  const int slice = t / D, i = t % D;
  float m = -INFINITY, l = 0.f, o = 0.f;
  for (int c0 = slice; c0 < nchunks; c0 += kCombBatch * S) {
    float mc[kCombBatch], lc[kCombBatch], oc[kCombBatch];
#pragma unroll
    for (int u = 0; u < kCombBatch; ++u) {
      const int c = min(c0 + u * S, nchunks - 1);
      const QD_GLOBAL float *pc = part + (size_t)c * (D + 2);
      mc[u] = pc[0];
      lc[u] = pc[1];
      oc[u] = pc[2 + i];
    }
    float mb = m;
#pragma unroll
    for (int u = 0; u < kCombBatch; ++u)
      if (c0 + u * S < nchunks) mb = fmaxf(mb, mc[u]);
    const float a = m == -INFINITY ? 0.f : __expf(m - mb);
    l *= a;
    o *= a;
#pragma unroll
    for (int u = 0; u < kCombBatch; ++u) {
      const float w = (c0 + u * S < nchunks && mc[u] != -INFINITY) ? __expf(mc[u] - mb) : 0.f;
      l = fmaf(lc[u], w, l);
      o = fmaf(oc[u], w, o);
    }
    m = mb;
  }
  sm[slice][i] = m;
  sl[slice][i] = l;
  so[slice][i] = o;
  __syncthreads();
  if (slice != 0) return;
  for (int q = 1; q < S; ++q) {
    const float m2 = sm[q][i], l2 = sl[q][i], o2 = so[q][i];
    const float mm = fmaxf(m, m2);
    const float a = m == -INFINITY ? 0.f : __expf(m - mm);
    const float b = m2 == -INFINITY ? 0.f : __expf(m2 - mm);
    l = l * a + l2 * b;
    o = o * a + o2 * b;
    m = mm;
  }
  out[i] = store16<F16>(o / l);
}

// The page's per-head RMSNorm (rounded to f16) and RoPE (rounded to f16) of
// this lane's 8 dimensions 8 * sub .. 8 * sub + 7 of one head; the head's
// other dimensions sit in the other lanes of the row slot (LPP lanes), the
// RoPE partner of dimension i (i +- d/2) in lane sub ^ LPP/2.  cs holds the
// cosine and sine of each pair's angle.
template <int D>
__device__ __forceinline__ void norm_rope8(float (&x)[8], const u32x4 wv, int sub, float eps,
                                           const float (*cs)[D / 2]) {
  constexpr int LPP = D / 8, HALF = D / 2;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
  for (int o = 1; o < LPP; o <<= 1) ss += __shfl_xor(ss, o, kWave);
  const float inv = 1.f / sqrtf(ss / (float)D + eps);
  const uint32_t we[4] = {wv.x, wv.y, wv.z, wv.w};
  float n[8], other[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    n[e] = f16_to_f32(f32_to_f16(x[e] * inv * bf16_to_f32((we[e >> 1] >> (16 * (e & 1))) & 0xffffu)));
#pragma unroll
  for (int e = 0; e < 8; ++e) other[e] = __shfl_xor(n[e], LPP / 2, kWave);
  const bool first = sub < LPP / 2;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int p = (8 * sub + e) % HALF;
    const float c = cs[0][p], s = cs[1][p];
    x[e] = f16_to_f32(f32_to_f16(first ? n[e] * c - other[e] * s : n[e] * c + other[e] * s));
  }
}

__device__ __forceinline__ u32x4 pack8_f16(const float (&v)[8]) {
  u32x4 r;
  r.x = (uint32_t)f32_to_f16(v[0]) | ((uint32_t)f32_to_f16(v[1]) << 16);
  r.y = (uint32_t)f32_to_f16(v[2]) | ((uint32_t)f32_to_f16(v[3]) << 16);
  r.z = (uint32_t)f32_to_f16(v[4]) | ((uint32_t)f32_to_f16(v[5]) << 16);
  r.w = (uint32_t)f32_to_f16(v[6]) | ((uint32_t)f32_to_f16(v[7]) << 16);
  return r;
}

// Chunk c of K/V head j for its G query heads.  With FINAL (a single chunk)
// the normalised output is stored; otherwise the partial (m, l, o[d]) goes to
// part[((j * G + h) * nchunks + c) * (d + 2) + {0: m, 1: l, 2..: o}]
// (nchunks = the grid's chunk count).  With pos_dev, the window is
// [0, *pos_dev + 1) and kv_start, length are ignored.  With QKR (device
// position, f16), q is raw: see AttentionQkRope.
template <int D, int G, bool F16, bool FINAL, bool QKR>
__global__ __launch_bounds__(kAttThreads) void attention_partial_kernel(
    const uint16_t *__restrict__ q_, const uint16_t *k_, const uint16_t *v_, int kv_heads,
    int kv_start, int length, int rows_per_wave, float scale, const int *__restrict__ pos_dev,
    int capacity, float *__restrict__ part, uint16_t *__restrict__ out_,
    const AttentionQkRope qkr) {
  // every argument loaded at the start (one scalar round trip): loaded where
  // first used, some would follow the position read as a second round trip
  __asm__ volatile("" ::"s"(q_), "s"(k_), "s"(v_), "s"(kv_heads), "s"(kv_start), "s"(length),
                   "s"(rows_per_wave), "s"(scale), "s"(pos_dev), "s"(capacity), "s"(part),
                   "s"(out_));
  __asm__ volatile("" ::"s"(qkr.k_src), "s"(qkr.v_src), "s"(qkr.q_w), "s"(qkr.k_w),
                   "s"(qkr.q_out), "s"(qkr.eps), "s"(qkr.theta), "s"(qkr.freq_ratio),
                   "s"(qkr.err));
  constexpr int LPP = D / 8;         // lanes per cached row
  constexpr int PPS = kWave / LPP;   // rows per wave load
  __shared__ float red[kAttWaves][G][10][LPP];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = blockIdx.y;          // K/V head
  const int c = blockIdx.x;          // chunk
  const int nchunks = gridDim.x;  // the partials' chunk stride
  const int sub = lane % LPP, grp = lane / LPP;
  if (pos_dev) {
    // window [0, position + 1) read from device memory; the grid covers the
    // whole cache and the chunks past the window exit
    const int pos = gp(pos_dev)[0];
    if (pos < 0 || pos >= capacity) {
      if (QKR && c == 0 && j == 0 && threadIdx.x == 0) atomicOr(qkr.err, 1u);
      return;
    }
    kv_start = 0;
    length = pos + 1;
    rows_per_wave = att_dev_rows_per_wave<D>(length, nchunks);
    if (c * kAttWaves * rows_per_wave >= length) return;
  }
  const QD_GLOBAL uint16_t *q = gp(q_);
  const QD_GLOBAL uint16_t *kc = gp(k_);
  const QD_GLOBAL uint16_t *vc = gp(v_);
  const size_t row = (size_t)kv_heads * D;  // elements per cache row

  // The rows of this wave: loads of the next rows are issued before the
  // current ones are computed (the first ones before q is prepared, after
  // the loads of the q/k prologue).
  const int t0 = kv_start + (c * kAttWaves + wave) * rows_per_wave;
  const int t1 = min(t0 + rows_per_wave, length);
  u32x4 kw[kAttUnroll], vw[kAttUnroll];
  bool valid[kAttUnroll];
  auto issue = [&](int tb) {
#pragma unroll
    for (int u = 0; u < kAttUnroll; ++u) {
      const int t = tb + u * PPS + grp;
      valid[u] = t < t1;
      const int tr = valid[u] ? t : t1 - 1;  // rows past the range re-read its last row
      const size_t off = (size_t)tr * row + (size_t)j * D + 8 * sub;
      kw[u] = *(const QD_GLOBAL u32x4 *)(kc + off);
      vw[u] = *(const QD_GLOBAL u32x4 *)(vc + off);
    }
  };
  // this lane's 8 dimensions of each query head, fp32, pre-scaled
  float qf[G][8];
  // QKR: the new K/V row of head j, for the chunk that holds it
  __shared__ __attribute__((aligned(16))) uint16_t knew[QKR ? D : 8], vnew[QKR ? D : 8];
  const int pos = length - 1;
  const bool mine = QKR && (pos - kv_start) / (kAttWaves * rows_per_wave) == c;
  if constexpr (QKR) {
    // The prologue's loads go first: waiting for them then leaves the cache
    // rows in flight, and the angles, norms and barriers below overlap them.
    __shared__ float cs[2][D / 2];
    u32x4 qraw[G], kraw, vraw;
    const u32x4 wq = *(const QD_GLOBAL u32x4 *)(gp(qkr.q_w) + 8 * sub);
#pragma unroll
    for (int h = 0; h < G; ++h)
      qraw[h] = *(const QD_GLOBAL u32x4 *)(q + (size_t)(j * G + h) * D + 8 * sub);
    const bool kwave = mine && wave == 0 && grp == 0;
    u32x4 wk = {0u, 0u, 0u, 0u};
    if (kwave) {
      kraw = *(const QD_GLOBAL u32x4 *)(gp(qkr.k_src) + (size_t)j * D + 8 * sub);
      vraw = *(const QD_GLOBAL u32x4 *)(gp(qkr.v_src) + (size_t)j * D + 8 * sub);
      wk = *(const QD_GLOBAL u32x4 *)(gp(qkr.k_w) + 8 * sub);
    }
    auto prologue = [&]() {
      if (threadIdx.x < D / 2) {
        // angle pos * theta^(-2i/d) and its reduction to [-pi, pi] in fp64
        // (a position of tens of thousands times the frequency needs it),
        // the sine and cosine of the reduced angle in fp32; theta^(-2i/d) is
        // (theta^(-2/d))^i by binary powering (i < 64: at most six squarings,
        // a relative error of about 1e-15)
        constexpr double kTwoPi = 6.283185307179586;
        double f = 1.0, b = qkr.freq_ratio;
#pragma unroll
        for (int e = 0; e < 6; ++e) {
          if ((threadIdx.x >> e) & 1) f *= b;
          b *= b;
        }
        const double ang = (double)pos * f;
        const float r = (float)(ang - kTwoPi * rint(ang / kTwoPi));
        float sn, cn;
        sincosf(r, &sn, &cn);
        cs[0][threadIdx.x] = cn;
        cs[1][threadIdx.x] = sn;
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < G; ++h) {
        unpack8<true>(qraw[h], qf[h]);
        norm_rope8<D>(qf[h], wq, sub, qkr.eps, cs);
      }
      // the rotated q rows, as the page's q buffer holds them after the RoPE
      // (one row slot of the first chunk's first wave stores them)
      if (qkr.q_out && c == 0 && wave == 0 && grp == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
          *(QD_GLOBAL u32x4 *)(gp(qkr.q_out) + (size_t)(j * G + h) * D + 8 * sub) =
              pack8_f16(qf[h]);
      }
      if (kwave) {
        float kx[8];
        unpack8<true>(kraw, kx);
        norm_rope8<D>(kx, wk, sub, qkr.eps, cs);
        const u32x4 kp = pack8_f16(kx);
        const size_t off = (size_t)pos * kv_heads * D + (size_t)j * D + 8 * sub;
        *(QD_GLOBAL u32x4 *)(gp((uint16_t *)k_) + off) = kp;
        *(QD_GLOBAL u32x4 *)(gp((uint16_t *)v_) + off) = vraw;
        *(u32x4 *)(knew + 8 * sub) = kp;
        *(u32x4 *)(vnew + 8 * sub) = vraw;
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[h][i] *= scale;
    };
    // in both branches: after a join of paths with different numbers of
    // loads in flight the memory waits would be counted for the path with
    // fewer, and the prologue would wait for the cache rows too (a wave's
    // barrier instructions count the same on either path)
    if (t0 < t1) {
      issue(t0);
      prologue();
    } else {
      prologue();
    }
  } else {
    if (t0 < t1) issue(t0);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      unpack8<F16>(*(const QD_GLOBAL u32x4 *)(q + (size_t)(j * G + h) * D + 8 * sub), qf[h]);
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[h][i] *= scale;
    }
  }
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
  }
  for (int tb = t0; tb < t1; tb += PPS * kAttUnroll) {
    if constexpr (QKR) {
      // the row this step appends: from LDS, not the cache being written
      if (mine) {
#pragma unroll
        for (int u = 0; u < kAttUnroll; ++u)
          if (tb + u * PPS + grp == pos) {
            kw[u] = *(const u32x4 *)(knew + 8 * sub);
            vw[u] = *(const u32x4 *)(vnew + 8 * sub);
          }
      }
    }
    float kf[kAttUnroll][8], vf[kAttUnroll][8];
    bool cv[kAttUnroll];
#pragma unroll
    for (int u = 0; u < kAttUnroll; ++u) {
      unpack8<F16>(kw[u], kf[u]);
      unpack8<F16>(vw[u], vf[u]);
      cv[u] = valid[u];
    }
    if (tb + PPS * kAttUnroll < t1) issue(tb + PPS * kAttUnroll);
#pragma unroll
    for (int u = 0; u < kAttUnroll; ++u) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(qf[h][i], kf[u][i], s);
        // the row's score: sum over its LPP lanes
#pragma unroll
        for (int w = 1; w < LPP; w <<= 1) s += __shfl_xor(s, w, kWave);
        if (!cv[u]) s = -INFINITY;
        const float mm = fmaxf(m[h], s);
        const float a = m[h] == -INFINITY ? 0.f : __expf(m[h] - mm);
        const float p = s == -INFINITY ? 0.f : __expf(s - mm);
        l[h] = l[h] * a + p;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] = fmaf(p, vf[u][i], o[h][i] * a);
        m[h] = mm;
      }
    }
  }
  // merge the row slots of the wave (lanes with the same sub)
#pragma unroll
  for (int w = LPP; w < kWave; w <<= 1) {
    float m2[G], l2[G], o2[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m2[h] = __shfl_xor(m[h], w, kWave);
      l2[h] = __shfl_xor(l[h], w, kWave);
#pragma unroll
      for (int i = 0; i < 8; ++i) o2[h][i] = __shfl_xor(o[h][i], w, kWave);
    }
    merge<G>(m, l, o, m2, l2, o2);
  }
  // merge the waves in LDS; the first row slot of wave 0 finishes the chunk
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      red[wave][h][0][sub] = m[h];
      red[wave][h][1][sub] = l[h];
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave][h][2 + i][sub] = o[h][i];
    }
  }
  __syncthreads();
  if (wave == 0) {
    if (grp == 0) {
      for (int w = 1; w < kAttWaves; ++w) {
        float m2[G], l2[G], o2[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          m2[h] = red[w][h][0][sub];
          l2[h] = red[w][h][1][sub];
#pragma unroll
          for (int i = 0; i < 8; ++i) o2[h][i] = red[w][h][2 + i][sub];
        }
        merge<G>(m, l, o, m2, l2, o2);
      }
      if (FINAL) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          uint32_t e[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            e[i] = (uint32_t)store16<F16>(o[h][2 * i] / l[h]) |
                   ((uint32_t)store16<F16>(o[h][2 * i + 1] / l[h]) << 16);
          u32x4 st;
          st.x = e[0];
          st.y = e[1];
          st.z = e[2];
          st.w = e[3];
          *(QD_GLOBAL u32x4 *)(gp(out_) + (size_t)(j * G + h) * D + 8 * sub) = st;
        }
      } else {
        QD_GLOBAL float *pp = gp(part);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          QD_GLOBAL float *dst = pp + ((size_t)(j * G + h) * nchunks + c) * (D + 2);
          if (sub == 0) {
            dst[0] = m[h];
            dst[1] = l[h];
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) dst[2 + 8 * sub + i] = o[h][i];
        }
      }
    }
  }
}

// out[h] from the nchunks partials of query head h (chunk stride `stride`),
// one workgroup per head; with pos_dev, nchunks follows from the window
// [0, *pos_dev + 1) (att_dev_rows_per_wave).
template <int D, bool F16>
__global__ __launch_bounds__(kAttThreads) void attention_combine_kernel(
    const float *__restrict__ part, int stride, int nchunks, const int *__restrict__ pos_dev,
    int capacity, int rows_per_wave, uint16_t *__restrict__ out) {
  const int h = blockIdx.x;
  if (pos_dev) {
    const int pos = gp(pos_dev)[0];
    if (pos < 0 || pos >= capacity) return;
    rows_per_wave = att_dev_rows_per_wave<D>(pos + 1, stride);
    nchunks = (pos + kAttWaves * rows_per_wave) / (kAttWaves * rows_per_wave);
  }
  combine_chunks<D, F16>(gp(part) + (size_t)h * stride * (D + 2), nchunks,
                            gp(out) + (size_t)h * D);
}

// Combine, then the o projection (decoder step).  Workgroup (s, j) merges
// the chunks of the G query heads of K/V head j exactly as
// attention_combine_kernel does (the same fp32 order, the row rounded to f16
// as the page stores it), then multiplies that row -- columns
// [j * G * D, (j + 1) * G * D) of the o projection's input -- by the same
// columns of rows [s * kCoRows, ...) of the affine-INT8 o weights:
//   opart[j][n] = sum_g (scale[n][g] * sum_k q[n][k] a[k] + bias[n][g] * sum_k a[k]).
// The o output of the page is f16(sum_j opart[j][n]), summed in j order by
// the next kernel's prologue; nothing is accumulated across workgroups.  The
// weight loads are issued first, so they are in flight during the combine.
constexpr int kCoThreads = 512;
constexpr int kCoPasses = 1;  // weight rows per lane (2 and 4 measured slower)

template <int D, int G>
__global__ __launch_bounds__(kCoThreads) void attention_combine_o_kernel(
    const float *__restrict__ part, int stride, const int *__restrict__ pos_dev, int capacity,
    int rows_per_wave, const uint8_t *__restrict__ wo, int rows, int cols,
    float *__restrict__ opart, uint16_t *__restrict__ attn_out) {
  // every argument loaded at the start (one scalar round trip)
  __asm__ volatile("" ::"s"(part), "s"(stride), "s"(pos_dev), "s"(capacity), "s"(rows_per_wave),
                   "s"(wo), "s"(rows), "s"(cols), "s"(opart), "s"(attn_out));
  constexpr int E = G * D;                           // elements of the K/V head's row slice
  constexpr int EW = E < kCoThreads ? E : kCoThreads;
  constexpr int SL = kCoThreads / EW;                // chunk slices side by side
  constexpr int EPT = E / EW;                        // elements per thread
  constexpr int LPR = E / 16;                        // lanes per weight row (16 codes each)
  constexpr int RPP = kCoThreads / LPR;              // rows per pass
  __shared__ float sm[SL][EW], sl[SL][EW], so[SL][EW];
  __shared__ __attribute__((aligned(16))) float av[E];
  const int t = threadIdx.x, j = blockIdx.y;
  const int u = t % LPR;
  const int groups = cols / 64;
  const QD_GLOBAL uint8_t *w = gp(wo);
  const QD_GLOBAL uint16_t *sc = (const QD_GLOBAL uint16_t *)(w + (size_t)rows * cols);
  const size_t boff = (size_t)rows * groups;
  const int c0 = j * E + 16 * u;                     // first column of this lane
  const int gi = c0 / 64;
  u32x4 q[kCoPasses];
  float scale[kCoPasses], bias[kCoPasses];
#pragma unroll
  for (int p = 0; p < kCoPasses; ++p) {
    const int n = min(blockIdx.x * (kCoPasses * RPP) + p * RPP + t / LPR, rows - 1);
    q[p] = *(const QD_GLOBAL u32x4 *)(w + (size_t)n * cols + c0);
    scale[p] = bf16_to_f32(sc[(size_t)n * groups + gi]);
    bias[p] = bf16_to_f32(sc[boff + (size_t)n * groups + gi]);
  }
  const int pos = gp(pos_dev)[0];
  if (pos < 0 || pos >= capacity) return;  // the first kernel has set the error word
  rows_per_wave = att_dev_rows_per_wave<D>(pos + 1, stride);
  const int nchunks = (pos + kAttWaves * rows_per_wave) / (kAttWaves * rows_per_wave);
  const int slice = t / EW, e0 = t % EW;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = e0 + k * EW;
    const int h = e / D, i = e % D;
    const QD_GLOBAL float *ph = gp(part) + (size_t)(j * G + h) * stride * (D + 2);
    float m = -INFINITY, l = 0.f, o = 0.f;
    for (int cb = slice; cb < nchunks; cb += kCombBatch * SL) {
      float mc[kCombBatch], lc[kCombBatch], oc[kCombBatch];
#pragma unroll
      for (int v = 0; v < kCombBatch; ++v) {
        const int c = min(cb + v * SL, nchunks - 1);
        const QD_GLOBAL float *pc = ph + (size_t)c * (D + 2);
        mc[v] = pc[0];
        lc[v] = pc[1];
        oc[v] = pc[2 + i];
      }
      float mb = m;
#pragma unroll
      for (int v = 0; v < kCombBatch; ++v)
        if (cb + v * SL < nchunks) mb = fmaxf(mb, mc[v]);
      const float a = m == -INFINITY ? 0.f : __expf(m - mb);
      l *= a;
      o *= a;
#pragma unroll
      for (int v = 0; v < kCombBatch; ++v) {
        const float wgt = (cb + v * SL < nchunks && mc[v] != -INFINITY) ? __expf(mc[v] - mb) : 0.f;
        l = fmaf(lc[v], wgt, l);
        o = fmaf(oc[v], wgt, o);
      }
      m = mb;
    }
    if constexpr (SL > 1) {
      sm[slice][e0] = m;
      sl[slice][e0] = l;
      so[slice][e0] = o;
      __syncthreads();
      if (slice == 0) {
        for (int r = 1; r < SL; ++r) {
          const float m2 = sm[r][e0], l2 = sl[r][e0], o2 = so[r][e0];
          const float mm = fmaxf(m, m2);
          const float a = m == -INFINITY ? 0.f : __expf(m - mm);
          const float b = m2 == -INFINITY ? 0.f : __expf(m2 - mm);
          l = l * a + l2 * b;
          o = o * a + o2 * b;
          m = mm;
        }
        av[e] = f16_to_f32(f32_to_f16(o / l));
      }
    } else {
      av[e] = f16_to_f32(f32_to_f16(o / l));
    }
  }
  __syncthreads();
  // the attention row of this K/V head's query heads, as the page's attn
  // buffer holds it (the first row block stores it)
  if (attn_out && blockIdx.x == 0)
    for (int e = t; e < E; e += kCoThreads) gp(attn_out)[(size_t)j * E + e] = f32_to_f16(av[e]);
  const float4 *ap = (const float4 *)(av + 16 * u);
  const float4 a0 = ap[0], a1 = ap[1], a2 = ap[2], a3 = ap[3];
  const float s16 = ((a0.x + a0.y) + (a0.z + a0.w)) + ((a1.x + a1.y) + (a1.z + a1.w)) +
                    ((a2.x + a2.y) + (a2.z + a2.w)) + ((a3.x + a3.y) + (a3.z + a3.w));
#pragma unroll
  for (int p = 0; p < kCoPasses; ++p) {
    const uint4 qq = {q[p].x, q[p].y, q[p].z, q[p].w};
    float v = fmaf(scale[p], dot16(qq, a0, a1, a2, a3), bias[p] * s16);
    v = group_sum<LPR>(v);
    const int n = blockIdx.x * (kCoPasses * RPP) + p * RPP + t / LPR;
    if (u == 0 && n < rows) gp(opart)[(size_t)j * rows + n] = v;
  }
}

template <int D, int G>
int combine_o_rows_per_wg() {
  return kCoPasses * (kCoThreads / (G * D / 16));
}

template <int D, int G, bool F16>
hipError_t launch_att(const AttentionArgs &a, hipStream_t stream) {
  // with a device position the chunk grid covers the whole cache
  const int window = a.pos_dev ? a.capacity : a.length - a.kv_start;
  const AttentionPlan p = attention_plan(a.kv_heads, window, D);
  if (p.nchunks < 1 || p.nchunks > attention_max_chunks(a.kv_heads)) return hipErrorInvalidValue;
  const AttentionQkRope none = {};
  if (p.nchunks == 1 && !a.pos_dev) {
    hipLaunchKernelGGL((attention_partial_kernel<D, G, F16, true, false>), dim3(1, a.kv_heads),
                       dim3(kAttThreads), 0, stream, a.q, a.k, a.v, a.kv_heads, a.kv_start,
                       a.length, p.rows_per_wave, a.scale, a.pos_dev, a.capacity, a.part, a.out,
                       none);
    return hipGetLastError();
  }
  if constexpr (F16) {
    if (a.qkr) {
      if (!a.pos_dev) return hipErrorInvalidValue;
      hipLaunchKernelGGL((attention_partial_kernel<D, G, true, false, true>),
                         dim3(p.nchunks, a.kv_heads), dim3(kAttThreads), 0, stream, a.q, a.k,
                         a.v, a.kv_heads, a.kv_start, a.length, p.rows_per_wave, a.scale,
                         a.pos_dev, a.capacity, a.part, a.out, *a.qkr);
    }
  }
  if (!a.qkr)
    hipLaunchKernelGGL((attention_partial_kernel<D, G, F16, false, false>),
                       dim3(p.nchunks, a.kv_heads), dim3(kAttThreads), 0, stream, a.q, a.k, a.v,
                       a.kv_heads, a.kv_start, a.length, p.rows_per_wave, a.scale, a.pos_dev,
                       a.capacity, a.part, a.out, none);
  else if (!F16)
    return hipErrorInvalidValue;
  if (a.wo) {
    if constexpr (F16) {
      if (!a.pos_dev || a.wo_cols != a.heads * D || a.wo_rows < 1) return hipErrorInvalidValue;
      const int rpw = combine_o_rows_per_wg<D, G>();
      hipLaunchKernelGGL((attention_combine_o_kernel<D, G>),
                         dim3((a.wo_rows + rpw - 1) / rpw, a.kv_heads), dim3(kCoThreads), 0,
                         stream, a.part, p.nchunks, a.pos_dev, a.capacity, p.rows_per_wave,
                         a.wo, a.wo_rows, a.wo_cols, a.opart, a.out);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((attention_combine_kernel<D, F16>), dim3(a.kv_heads * G),
                     dim3(kAttThreads), 0, stream, a.part, p.nchunks, p.nchunks, a.pos_dev,
                     a.capacity, p.rows_per_wave, a.out);
  return hipGetLastError();
}

template <int D, bool F16>
hipError_t launch_att_g(const AttentionArgs &a, hipStream_t stream) {
  switch (a.heads / a.kv_heads) {
    case 1: return launch_att<D, 1, F16>(a, stream);
    case 2: return launch_att<D, 2, F16>(a, stream);
    case 4: return launch_att<D, 4, F16>(a, stream);
    default: return launch_att<D, 8, F16>(a, stream);
  }
}

}  // namespace

// Chunk partials of attention_decode_noalloc: a file-scope device array (one
// copy per device, alive until the process ends) instead of a caller
// workspace.  Host code never names it: its address on the current device
// comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kNoallocScratchBytes = 4u << 20;
static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch[kMaxScratchDevices];
}  // namespace

size_t attention_noalloc_scratch_bytes() { return kNoallocScratchBytes; }

hipError_t attention_noalloc_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    // the current device's copy of the array (two threads racing here get
    // the same address)
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

AttentionPlan attention_plan(int64_t kv_heads, int64_t window, int head_dim) {
  // whole loads of rows per wave, about kAttTargetWgs workgroups in all
  const int64_t step = (int64_t)(kWave / (head_dim / 8)) * kAttUnroll;
  const int64_t want = (kAttTargetWgs + kv_heads - 1) / kv_heads;
  int64_t rpw = (window + want * kAttWaves - 1) / (want * kAttWaves);
  // a short window is one chunk: one launch beats a second one for the merge
  if (window <= kAttWaves * kAttSingleRowsPerWave) rpw = (window + kAttWaves - 1) / kAttWaves;
  rpw = (rpw + step - 1) / step * step;
  if (rpw < step) rpw = step;
  AttentionPlan p;
  p.rows_per_wave = (int)rpw;
  p.nchunks = (int)((window + rpw * kAttWaves - 1) / (rpw * kAttWaves));
  return p;
}

int64_t attention_max_chunks(int64_t kv_heads) {
  // nchunks = ceil(window / (kAttWaves * rpw)) with kAttWaves * rpw >= window / want
  return (kAttTargetWgs + kv_heads - 1) / kv_heads;
}

hipError_t launch_attention_decode(const AttentionArgs &a, hipStream_t stream) {
  if (a.head_dim == 64)
    return a.f16 ? launch_att_g<64, true>(a, stream) : launch_att_g<64, false>(a, stream);
  return a.f16 ? launch_att_g<128, true>(a, stream) : launch_att_g<128, false>(a, stream);
}

}  // namespace qd
