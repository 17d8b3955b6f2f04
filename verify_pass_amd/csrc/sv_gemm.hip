// Weight-streaming GEMM over the stacked verify tokens, gfx950.
//
// Y^T[N][T] = W[N][K] * X^T: weight rows are the MFMA's M side and tokens its
// N side.  One read of the weights serves every stacked token of every
// sequence -- the single weight stream a verification pass is built around.
//
// Work unit = one wave: 32 weight rows (two 16-row MFMA tiles) x up to 64
// tokens x one split of K.  The unit streams its weight rows straight from HBM
// into registers with a rolling prefetch and reads the (small, L2-resident)
// token rows directly as MFMA B operands: no LDS staging, no barriers, so the
// four waves of a workgroup run independently and keep memory busy.
//
// The two tiles of a unit are chosen so that every epilogue is lane-local:
//   QKV     tile 0 = rotation-pair firsts, tile 1 = their partners (i + hd/2):
//           RMSNorm scale, RoPE, q to a staging buffer, k/v appended to caches
//   SWIGLU  tile 0 = gate rows, tile 1 = the matching up rows: silu(g) * u
//   RESID   + residual (O and down projections)
//   LOGITS  fp32 logits and per-(32 rows, token) softmax statistics
// RMSNorm only needs a per-token scale r_t = 1/sqrt(mean(x^2) + eps):
// (r_t x) W = r_t (x W), so it is applied in the epilogue from sums of squares
// of the token operand the unit already loads.
//
// K splits: when there are too few row groups to occupy the chip, units also
// split K.  Each split stores its fp32 partial tile with device-scope (sc1)
// stores, waits for them to complete and bumps a per-tile counter; the split
// that arrives last reads the partials back with device-scope loads, adds
// them in split order (bitwise repeatable) and runs the epilogue.  No
// cache-wide fence is involved.
#include "sv_common.h"

namespace sv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;

// Raw per-lane payload of one K step for one 16-row tile.
template <int WT> struct WStep;
template <> struct WStep<WT_BF16> { uint4 v[2]; };
template <> struct WStep<WT_F32> { uint4 v[4]; };
template <> struct WStep<WT_INT4> { uint4 v; uint32_t s; };

template <int WT> constexpr int kstep() { return WT == WT_INT4 ? 128 : 64; }

// Lane (row, gq) of step ks holds, for MFMA m, reduction indices
//   bf16 : ks*64  + 32m + 8gq + [0, 8)      (each instruction: 64 contiguous
//          bytes per row across the four lane groups)
//   int4 : ks*128 + 32gq + 8m + [0, 8)      (one 16-byte load per lane)
//   fp32 : ks*64  + 16gq + 8m + [0, 8)
// and the token operand holds the same indices for its token.
template <int WT>
__device__ __forceinline__ WStep<WT> load_w(const void *w, const uint16_t *sc, int row, int K, int ks,
                                           int gq) {
  WStep<WT> r;
  if constexpr (WT == WT_BF16) {
    const uint16_t *b = static_cast<const uint16_t *>(w) + (size_t)row * K + ks * 64 + 8 * gq;
    r.v[0] = *reinterpret_cast<const uint4 *>(b);
    r.v[1] = *reinterpret_cast<const uint4 *>(b + 32);
  } else if constexpr (WT == WT_F32) {
    const float *b = static_cast<const float *>(w) + (size_t)row * K + ks * 64 + 16 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = *reinterpret_cast<const uint4 *>(b + 4 * i);
  } else {
    const uint32_t *b = static_cast<const uint32_t *>(w) + (size_t)row * (K / 8) + ks * 16 + 4 * gq;
    r.v = *reinterpret_cast<const uint4 *>(b);
    r.s = sc[(size_t)row * (K / 32) + ks * 4 + gq];
  }
  return r;
}

// Token operand of one step: lane (token, gq) holds the step's reduction
// indices in the same order as the weight operand (KS/4 bf16 values).
template <int WT> struct XStep;
template <> struct XStep<WT_BF16> { uint4 v[2]; };
template <> struct XStep<WT_F32> { uint4 v[2]; };
template <> struct XStep<WT_INT4> { uint4 v[4]; };

template <int WT>
__device__ __forceinline__ XStep<WT> load_x(const uint16_t *xrow, int ks, int gq) {
  XStep<WT> r;
  if constexpr (WT == WT_BF16) {
    const uint16_t *b = xrow + ks * 64 + 8 * gq;
    r.v[0] = *reinterpret_cast<const uint4 *>(b);
    r.v[1] = *reinterpret_cast<const uint4 *>(b + 32);
  } else {
    constexpr int KS = kstep<WT>();
    const uint16_t *b = xrow + ks * KS + (KS / 4) * gq;
#pragma unroll
    for (int i = 0; i < (KS / 32); ++i) r.v[i] = *reinterpret_cast<const uint4 *>(b + 8 * i);
  }
  return r;
}

// int4 word (8 codes, offset by 8) times the group scale, to bf16.
__device__ __forceinline__ bf16x8 dequant8(uint32_t word, float s) {
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = static_cast<float>(static_cast<int>((word >> (4 * e)) & 15u) - 8) * s;
    h[e] = f2bf(v);
  }
  return as_bf16x8(uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                         h[6] | (h[7] << 16)});
}

// fp32 x8 -> (hi, lo) bf16 pairs with hi + lo == v to about 2^-17 relative.
__device__ __forceinline__ void split8(const uint4 &a, const uint4 &b, bf16x8 &hi, bf16x8 &lo) {
  const float f[8] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z),
                      __uint_as_float(a.w), __uint_as_float(b.x), __uint_as_float(b.y),
                      __uint_as_float(b.z), __uint_as_float(b.w)};
  uint32_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = f2bf(f[e]);
    l[e] = f2bf(f[e] - bf2f(static_cast<uint16_t>(h[e])));
  }
  hi = as_bf16x8(uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)});
  lo = as_bf16x8(uint4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)});
}

__device__ __forceinline__ float sumsq8(const uint4 &v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = __uint_as_float(w[i] << 16), b = __uint_as_float(w[i] & 0xFFFF0000u);
    s += a * a;
    s += b * b;
  }
  return s;
}

// Physical (matrix, row) of row r of tile `tile` in 32-row group g.
// Returns false past the end of the matrix (the lane then streams row 0 and
// its results are dropped).
__device__ __forceinline__ bool map_row(const GemmParams &p, int g, int tile, int r, int &m, int &pr) {
  int n;
  if (p.rowmap == RM_SWIGLU) {
    const int f = g * 16 + r;
    if (f >= p.mat[0].rows) return false;
    m = tile;
    pr = f;
    return true;
  }
  if (p.rowmap == RM_ROPE_PAIRS) {
    const int gph = p.hd / 32;  // groups per head
    const int head = g / gph, c = g - head * gph;
    n = head * p.hd + tile * (p.hd / 2) + 16 * c + r;
  } else {
    n = g * 32 + tile * 16 + r;
  }
  if (n >= p.N) return false;
  int k = 0;
  while (k < p.nmat - 1 && n >= p.mat[k].rows) {
    n -= p.mat[k].rows;
    ++k;
  }
  m = k;
  pr = n;
  return true;
}

// Bijective remap of the dispatch index so that consecutive logical
// workgroups run on the same XCD (dispatch is round-robin over the 8 XCDs).
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  const int q = nwg / 8, r = nwg % 8;
  const int x = wg % 8, k = wg / 8;
  return x * q + min(x, r) + k;
}

__device__ __forceinline__ void store_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this wave's outstanding vector memory operations have completed
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Sequence and position of stacked token t (each lane passes its own t).
// The token map is the prefix sum of gamma_i + 1, built 64 sequences at a
// time with a wave scan; the owner of t is the last sequence starting <= t.
__device__ inline void token_pos(const GemmParams &p, int t, int lane, int &seq, int &pos) {
  int base = 0, found = 0, fstart = 0;
  for (int c0 = 0; c0 < p.B; c0 += 64) {
    const int i = c0 + lane;
    const int v = i < p.B ? p.gamma[i] + 1 : 0;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    const int start = base + inc - v;
    const int n = min(64, p.B - c0);
    for (int j = 0; j < n; ++j) {
      const int sj = __shfl(start, j);
      if (sj <= t) {
        found = c0 + j;
        fstart = sj;
      }
    }
    base += __shfl(inc, 63);
  }
  seq = found;
  pos = p.kv_len[seq] + (t - fstart);
}

template <int WT, int TT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmParams p) {
  constexpr int MPS = WT == WT_BF16 ? 2 : 4;      // MFMAs per step per tile pair member
  constexpr int P = TT <= 2 ? 4 : 3;              // prefetch depth in K steps

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gq = lane >> 4, l16 = lane & 15;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int unit = wg * kWaves + wave;
  const int ngrp = p.nblk;
  const int nunits = ngrp * p.splits * p.ntblk;
  if (unit >= nunits) return;
  const int grp = unit % ngrp;
  const int rest = unit / ngrp;
  const int split = rest % p.splits;
  const int tb = rest / p.splits;
  const int t0 = tb * TT * 16;
  const int s0 = (int)((long long)split * p.ksteps / p.splits);
  const int s1 = (int)((long long)(split + 1) * p.ksteps / p.splits);
  const int nsteps = s1 - s0;

  // weight rows this lane streams (one per tile)
  const void *wb[2];
  const uint16_t *sb[2];
  int prow[2];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    int mi = 0, pr = 0;
    if (!map_row(p, grp, tile, l16, mi, pr)) { mi = 0; pr = 0; }
    wb[tile] = p.mat[mi].w;
    sb[tile] = p.mat[mi].s;
    prow[tile] = pr;
  }
  // token rows this lane reads (clamped; results of padding tokens are dropped)
  const uint16_t *xr[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) xr[tt] = p.x + (size_t)min(t0 + tt * 16 + l16, p.T - 1) * p.K;

  floatx4 acc[2][TT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[a][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float ss[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) ss[tt] = 0.f;

  WStep<WT> wbuf[P][2];
  XStep<WT> xbuf[P][TT];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int st = s0 + min(j, nsteps - 1);
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) wbuf[j][tile] = load_w<WT>(wb[tile], sb[tile], prow[tile], p.K, st, gq);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) xbuf[j][tt] = load_x<WT>(xr[tt], st, gq);
  }

  for (int base = 0; base < nsteps; base += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      if (base + j < nsteps) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          if (p.norm) {
#pragma unroll
            for (int i = 0; i < (kstep<WT>() / 32); ++i) ss[tt] += sumsq8(xbuf[j][tt].v[i]);
          }
#pragma unroll
          for (int tile = 0; tile < 2; ++tile) {
            if constexpr (WT == WT_BF16) {
#pragma unroll
              for (int m = 0; m < 2; ++m)
                acc[tile][tt] = mfma16x16x32(as_bf16x8(wbuf[j][tile].v[m]), as_bf16x8(xbuf[j][tt].v[m]), acc[tile][tt]);
            } else if constexpr (WT == WT_INT4) {
              const float s = bf2f(static_cast<uint16_t>(wbuf[j][tile].s));
              const uint32_t wv[4] = {wbuf[j][tile].v.x, wbuf[j][tile].v.y, wbuf[j][tile].v.z, wbuf[j][tile].v.w};
#pragma unroll
              for (int m = 0; m < 4; ++m)
                acc[tile][tt] = mfma16x16x32(dequant8(wv[m], s), as_bf16x8(xbuf[j][tt].v[m]), acc[tile][tt]);
            } else {
#pragma unroll
              for (int m = 0; m < 2; ++m) {
                bf16x8 hi, lo;
                split8(wbuf[j][tile].v[2 * m], wbuf[j][tile].v[2 * m + 1], hi, lo);
                acc[tile][tt] = mfma16x16x32(hi, as_bf16x8(xbuf[j][tt].v[m]), acc[tile][tt]);
                acc[tile][tt] = mfma16x16x32(lo, as_bf16x8(xbuf[j][tt].v[m]), acc[tile][tt]);
              }
            }
          }
        }
      }
      const int nx = s0 + min(base + j + P, nsteps - 1);
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) wbuf[j][tile] = load_w<WT>(wb[tile], sb[tile], prow[tile], p.K, nx, gq);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) xbuf[j][tt] = load_x<WT>(xr[tt], nx, gq);
    }
  }
  (void)MPS;

  // sums of squares of this split's token slices: add the four lane groups
  if (p.norm) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      ss[tt] += __shfl_xor(ss[tt], 16);
      ss[tt] += __shfl_xor(ss[tt], 32);
    }
  }

  // ---- K-split reduction ----------------------------------------------------
  if (p.splits > 1) {
    constexpr int TILE = 2 * TT * 4 * 64 + TT * 64;  // partial values + sums of squares
    const size_t tile_id = (size_t)tb * ngrp + grp;
    float *mine = p.partial + ((size_t)split * ngrp * p.ntblk + tile_id) * TILE;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) store_dev(mine + ((a * TT + tt) * 4 + i) * 64 + lane, acc[a][tt][i]);
    if (p.norm) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) store_dev(mine + 2 * TT * 4 * 64 + tt * 64 + lane, ss[tt]);
    }
    wait_vmem();
    int old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(p.counters + tile_id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0);
    if (old != p.splits - 1) return;
    if (lane == 0) __hip_atomic_store(p.counters + tile_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[a][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) ss[tt] = 0.f;
    for (int sp = 0; sp < p.splits; ++sp) {
      const float *src = p.partial + ((size_t)sp * ngrp * p.ntblk + tile_id) * TILE;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[a][tt][i] += load_dev(src + ((a * TT + tt) * 4 + i) * 64 + lane);
      if (p.norm) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) ss[tt] += load_dev(src + 2 * TT * 4 * 64 + tt * 64 + lane);
      }
    }
  }

  // per-token RMSNorm scale (lane's token is t0 + tt*16 + l16)
  float rs[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) rs[tt] = p.norm ? 1.f / sqrtf(ss[tt] / static_cast<float>(p.K) + p.eps) : 1.f;

  // ---- fused epilogues (lane-local) -----------------------------------------
  if (p.epi == EPI_RESID) {
    uint16_t *out = static_cast<uint16_t *>(p.out);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = t0 + tt * 16 + l16;
      if (t >= p.T) continue;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = grp * 32 + a * 16 + 4 * gq + i;
          if (n < p.N) {
            const size_t o = (size_t)t * p.ldo + n;
            out[o] = f2bf(acc[a][tt][i] * rs[tt] + bf2f(p.resid[o]));
          }
        }
    }
  } else if (p.epi == EPI_SWIGLU) {
    uint16_t *out = static_cast<uint16_t *>(p.out);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = t0 + tt * 16 + l16;
      if (t >= p.T) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = grp * 16 + 4 * gq + i;
        if (f < p.mat[0].rows) {
          const float g = acc[0][tt][i] * rs[tt], u = acc[1][tt][i] * rs[tt];
          const float sig = 1.f / (1.f + __builtin_amdgcn_exp2f(-g * kLog2e));
          out[(size_t)t * p.ldo + f] = f2bf(g * sig * u);
        }
      }
    }
  } else if (p.epi == EPI_LOGITS) {
    float *out = static_cast<float *>(p.out);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = t0 + tt * 16 + l16;
      float v[8];
      float m = -INFINITY;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = grp * 32 + a * 16 + 4 * gq + i;
          v[a * 4 + i] = n < p.N ? acc[a][tt][i] * rs[tt] : -INFINITY;
          m = fmaxf(m, v[a * 4 + i]);
          if (t < p.T && n < p.N) out[(size_t)t * p.ldo + n] = v[a * 4 + i];
        }
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += __builtin_amdgcn_exp2f((v[e] - m) * kLog2e);
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (gq == 0 && t < p.T) {
        float *st = p.stats + ((size_t)grp * p.T + t) * 2;
        st[0] = m;
        st[1] = s;
      }
    }
  } else {  // EPI_QKV: tile 0 holds pair firsts i, tile 1 the partners i + hd/2
    const int gph = p.hd / 32;
    const int head = grp / gph, c = grp - head * gph;
    const int half = p.hd / 2;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = t0 + tt * 16 + l16;
      int seq = 0, pos = 0;
      token_pos(p, min(t, p.T - 1), lane, seq, pos);
      if (t >= p.T) continue;
      const bool kv_ok = pos >= 0 && pos < p.kv_cap;
      if (head >= p.hq && !kv_ok) {
        set_err(p.err, SV_DEV_ERR_KV_OVERFLOW);
        continue;
      }
      float ra[4], rb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int fi = 16 * c + 4 * gq + e;  // rotation pair (fi, fi + hd/2)
        const float a = acc[0][tt][e] * rs[tt], b = acc[1][tt][e] * rs[tt];
        if (head < p.hq + p.hkv) {
          const double inv = pow(static_cast<double>(p.rope_theta), -2.0 * fi / p.hd);
          double sn, cs;
          sincos(static_cast<double>(pos) * inv, &sn, &cs);
          const float cf = static_cast<float>(cs), sf = static_cast<float>(sn);
          ra[e] = a * cf - b * sf;
          rb[e] = b * cf + a * sf;
        } else {
          ra[e] = a;
          rb[e] = b;
        }
      }
      const int fi0 = 16 * c + 4 * gq;
      if (head < p.hq) {
        uint16_t *q = p.qbuf + ((size_t)t * p.hq + head) * p.hd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          q[fi0 + e] = f2bf(ra[e]);
          q[fi0 + half + e] = f2bf(rb[e]);
        }
      } else if (head < p.hq + p.hkv) {
        uint16_t *k = static_cast<uint16_t *>(p.kc[seq]) + ((size_t)(head - p.hq) * p.kv_cap + pos) * p.hd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k[fi0 + e] = f2bf(ra[e]);
          k[fi0 + half + e] = f2bf(rb[e]);
        }
      } else {
        uint16_t *v = static_cast<uint16_t *>(p.vc[seq]) + (size_t)(head - p.hq - p.hkv) * p.hd * p.kv_cap;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[(size_t)(fi0 + e) * p.kv_cap + pos] = f2bf(ra[e]);
          v[(size_t)(fi0 + half + e) * p.kv_cap + pos] = f2bf(rb[e]);
        }
      }
    }
  }
}

template <int WT, int TT>
hipError_t launch_tt(const GemmParams &p, hipStream_t s, int trace_class) {
  const int nunits = p.nblk * p.splits * p.ntblk;
  const int nwg = (nunits + kWaves - 1) / kWaves;
  trace_before(trace_class, s);
  hipLaunchKernelGGL((gemm_kernel<WT, TT>), dim3(nwg), dim3(kThreads), 0, s, p);
  trace_after(trace_class, s);
  return hipGetLastError();
}

template <int WT>
hipError_t launch_wt(const GemmParams &p, int tt, hipStream_t s, int tc) {
  switch (tt) {
    case 1: return launch_tt<WT, 1>(p, s, tc);
    case 2: return launch_tt<WT, 2>(p, s, tc);
    case 3: return launch_tt<WT, 3>(p, s, tc);
    default: return launch_tt<WT, 4>(p, s, tc);
  }
}

}  // namespace

hipError_t launch_gemm(const GemmParams &p, int wtype, int tok_tiles, hipStream_t s,
                       int trace_class) {
  if (wtype == WT_BF16) return launch_wt<WT_BF16>(p, tok_tiles, s, trace_class);
  if (wtype == WT_INT4) return launch_wt<WT_INT4>(p, tok_tiles, s, trace_class);
  return launch_wt<WT_F32>(p, tok_tiles, s, trace_class);
}

size_t gemm_partial_floats(int ngroups, int splits, int ntblk, int tok_tiles) {
  if (splits <= 1) return 0;
  return (size_t)splits * ngroups * ntblk * (2 * tok_tiles * 4 * 64 + tok_tiles * 64);
}

}  // namespace sv
