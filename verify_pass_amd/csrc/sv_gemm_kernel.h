// Weight-streaming GEMM kernel templates, instantiated once per weight type
// (sv_gemm_bf16.hip, sv_gemm_int4.hip, sv_gemm_f32.hip) so that the three
// translation units compile in parallel.
#pragma once
#include <type_traits>
#include <utility>

#include "sv_common.h"

namespace sv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Raw per-lane payload of one K step for one 16-row tile.
template <int WT> struct WStep;
template <> struct WStep<WT_BF16> { uint4 v[2]; };
template <> struct WStep<WT_F32> { uint4 v[4]; };
template <> struct WStep<WT_INT4> { uint4 v; uint32_t s; };

template <int WT> constexpr int kstep() { return WT == WT_INT4 ? 128 : 64; }

// One-wave-per-unit launches share the token operand of a K step among the
// workgroup's units through LDS: xfrags 16-byte fragments per lane and token
// tile (the XStep payload), in a ring of two groups of G steps.
template <int WT> constexpr int xfrags() { return WT == WT_INT4 ? 4 : 2; }
template <int WT, int TT, int G> constexpr int xl_bytes() { return 2 * G * TT * xfrags<WT>() * 1024; }
constexpr int kXlMax = 64 * 1024;
// Element offset of fragment m of lane group gq inside a token row's K step.
template <int WT> __device__ __forceinline__ int xoff(int m, int gq) {
  return WT == WT_BF16 ? 32 * m + 8 * gq : WT == WT_INT4 ? 32 * gq + 8 * m : 16 * gq + 8 * m;
}
typedef __attribute__((address_space(3))) void lds_void;
// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16 l (lds wave-uniform).
__device__ __forceinline__ void load_lds16(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void load_lds16(const void *g, lds_void *lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Streaming (non-temporal) 16-byte load: weights are read once per pass and
// should not evict the token operand from L2.
__device__ __forceinline__ uint4 ld_nt(const void *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return __builtin_bit_cast(uint4, v);
}
// Plain 16-byte load through the vector type (keeps staging arrays in registers).
__device__ __forceinline__ uint4 ld_v4(const void *p) {
  return __builtin_bit_cast(uint4, *reinterpret_cast<const u32x4 *>(p));
}

// Per-lane weight stream of one 16-row tile.
// Lane (row, gq) of step ks holds, for MFMA m, reduction indices
//   bf16 : ks*64  + 32m + 8gq + [0, 8)
//   int4 : ks*128 + 32gq + 8m + [0, 8)      (one 16-byte word group per lane)
//   fp32 : ks*64  + 16gq + 8m + [0, 8)
// and the token operand holds the same indices for its token.
// Row-major [N][K] storage: each load instruction reads 16 rows x 64 bytes.
// Packed storage (see sv_pack_matrix): the 16-row tile's fragments for one
// step are contiguous in lane order, so each load instruction reads 1 KiB of
// contiguous memory and a tile's whole K range is one sequential stream.
template <int WT>
struct WSrc {
  const unsigned char *p;   // lane's base address for step 0
  const uint16_t *s;        // int4 scales, lane's base for step 0
  int step_bytes;           // byte advance per K step
  int s_step;               // scale advance (elements) per K step
  int m_off;                // byte offset of the second fragment (bf16)
};

template <int WT>
__device__ __forceinline__ WSrc<WT> make_src(const GemmMat &mat, int row, int tile_row0, int K,
                                             int ksteps, int packed, int lane, int gq) {
  WSrc<WT> w;
  if (packed) {
    // step-major: K step s of 32-row group g at (s * ng + g); tile a within it
    const size_t g = (size_t)(tile_row0 / 32);
    const int ng = (mat.rows + 31) / 32;
    const int a = (tile_row0 / 16) & 1;
    if constexpr (WT == WT_INT4) {
      w.p = static_cast<const unsigned char *>(mat.w) + ((g * 2 + a) * 64 + lane) * 16;
      w.s = mat.s + (g * 2 + a) * 64 + lane;
      w.step_bytes = ng * 2 * 64 * 16;
      w.s_step = ng * 2 * 64;
      w.m_off = 0;
    } else {
      w.p = static_cast<const unsigned char *>(mat.w) + ((g * 2 + a) * 128 + lane) * 16;
      w.s = nullptr;
      w.step_bytes = ng * 2 * 128 * 16;
      w.s_step = 0;
      w.m_off = 64 * 16;
    }
  } else {
    if constexpr (WT == WT_BF16) {
      w.p = static_cast<const unsigned char *>(mat.w) + ((size_t)row * K + 8 * gq) * 2;
      w.step_bytes = 128;
      w.m_off = 64;
      w.s = nullptr;
      w.s_step = 0;
    } else if constexpr (WT == WT_INT4) {
      w.p = static_cast<const unsigned char *>(mat.w) + ((size_t)row * (K / 8) + 4 * gq) * 4;
      w.step_bytes = 64;
      w.m_off = 0;
      w.s = mat.s + (size_t)row * (K / 32) + gq;
      w.s_step = 4;
    } else {
      w.p = static_cast<const unsigned char *>(mat.w) + ((size_t)row * K + 16 * gq) * 4;
      w.step_bytes = 256;
      w.m_off = 0;
      w.s = nullptr;
      w.s_step = 0;
    }
  }
  return w;
}

template <int WT>
__device__ __forceinline__ WStep<WT> load_w(const WSrc<WT> &w, int ks) {
  WStep<WT> r;
  const unsigned char *b = w.p + (size_t)ks * w.step_bytes;
  if constexpr (WT == WT_BF16) {
    r.v[0] = ld_nt(b);
    r.v[1] = ld_nt(b + w.m_off);
  } else if constexpr (WT == WT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = ld_nt(b + 16 * i);
  } else {
    r.v = ld_nt(b);
    r.s = w.s[(size_t)ks * w.s_step];
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

// a & m through one v_and_b32 the compiler cannot see into: it then
// converts each masked byte with v_cvt_f32_ubyte{0..3} instead of first
// re-extracting every 4-bit field from the original word
__device__ __forceinline__ uint32_t and_opaque(uint32_t a, uint32_t m) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(m), "v"(a));
  return r;
}

// int4 word (8 codes, offset by 8) times the group scale, to bf16.  The
// nibbles are unpacked bytewise (one mask for the even, a shift and mask for
// the odd ones, each byte then converted to fp32 directly); (code - 8) * s is
// one fma from the unsigned nibble, exact in fp32 (a 4-bit times an 8-bit
// significand), and pairs are rounded to bf16 by one conversion each:
// 23 VALU operations per 8 weights.
__device__ __forceinline__ bf16x8 dequant8(uint32_t word, float s) {
  const uint32_t ev = and_opaque(word, 0x0F0F0F0Fu), od = and_opaque(word >> 4, 0x0F0F0F0Fu);
  const float m8 = -8.f * s;
  uint32_t h[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float fe = static_cast<float>((ev >> (8 * b)) & 0xFFu);  // nibble 2b
    const float fo = static_cast<float>((od >> (8 * b)) & 0xFFu);  // nibble 2b + 1
    h[b] = pack_bf16x2(fmaf(fe, s, m8), fmaf(fo, s, m8));
  }
  return as_bf16x8(uint4{h[0], h[1], h[2], h[3]});
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

// One K step of one 16-row tile times one token fragment.
template <int WT>
__device__ __forceinline__ void mma_tile(const WStep<WT> &w, const XStep<WT> &x, floatx4 &acc) {
  if constexpr (WT == WT_BF16) {
#pragma unroll
    for (int m = 0; m < 2; ++m) acc = mfma16x16x32(as_bf16x8(w.v[m]), as_bf16x8(x.v[m]), acc);
  } else if constexpr (WT == WT_INT4) {
    const float s = bf2f(static_cast<uint16_t>(w.s));
    const uint32_t wv[4] = {w.v.x, w.v.y, w.v.z, w.v.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) acc = mfma16x16x32(dequant8(wv[m], s), as_bf16x8(x.v[m]), acc);
  } else {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bf16x8 hi, lo;
      split8(w.v[2 * m], w.v[2 * m + 1], hi, lo);
      acc = mfma16x16x32(hi, as_bf16x8(x.v[m]), acc);
      acc = mfma16x16x32(lo, as_bf16x8(x.v[m]), acc);
    }
  }
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

// Four consecutive bf16 as one 8-byte access (the lane's four rows 4gq..4gq+3
// of a tile are consecutive output columns).
__device__ __forceinline__ void st_bf16x4(uint16_t *o, const float (&v)[4]) {
  *reinterpret_cast<uint2 *>(o) = make_uint2(f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16),
                                             f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16));
}

// RMSNorm scale of the operand rows for this lane's tokens (t0 + 16 tt + l16):
// precomputed scales, or sums of squares left in partials by the producer,
// or 1.
template <int TT>
__device__ __forceinline__ void token_scales(const GemmParams &p, int t0, int gq, int l16, float (&rs)[TT]) {
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int t = min(t0 + tt * 16 + l16, p.T - 1);
    if (p.rnorm) {
      rs[tt] = p.rnorm[t];
    } else if (p.rparts) {
      // lane group gq adds partials gq, gq+4, ... of its token; then the groups
      float s = 0.f;
      const float *pr = p.rparts + (size_t)t * p.nparts;
#pragma unroll 32
      for (int g = gq; g < p.nparts; g += 4) s += pr[g];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      rs[tt] = 1.f / sqrtf(s / static_cast<float>(p.K) + p.eps);
    } else {
      rs[tt] = 1.f;
    }
  }
}

template <int TT, int EPI>
__device__ __forceinline__ void epilogue_rs(const GemmParams &p, floatx4 (&acc)[2][TT], int grp, int t0, int gq,
                                            int l16, const float (&rs)[TT]);

// The fused epilogue of one 32-row group: acc[a][tt] holds rows (group grp,
// tile a, 4*gq + i) x token t0 + 16*tt + l16 of this lane.
template <int TT, int EPI>
__device__ __forceinline__ void epilogue(const GemmParams &p, floatx4 (&acc)[2][TT], int grp, int t0, int gq,
                                         int l16) {
  float rs[TT];
  token_scales<TT>(p, t0, gq, l16, rs);
  epilogue_rs<TT, EPI>(p, acc, grp, t0, gq, l16, rs);
}

template <int TT, int EPI>
__device__ __forceinline__ void epilogue_rs(const GemmParams &p, floatx4 (&acc)[2][TT], int grp, int t0, int gq,
                                            int l16, const float (&rs)[TT]) {
  // ---- fused epilogues (lane-local) -----------------------------------------
  // Each lane holds, per tile, four consecutive output columns (rows 4gq..4gq+3
  // of the tile): written as one 8- or 16-byte access when the row stride keeps
  // them aligned and all four exist.
  const bool vec = (p.ldo & 3) == 0;
  if constexpr (EPI == EPI_RESID) {
    uint16_t *out = static_cast<uint16_t *>(p.out);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = t0 + tt * 16 + l16;
      float sq = 0.f;  // this lane's share of the output row's sum of squares
      if (t < p.T) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int n0 = grp * 32 + a * 16 + 4 * gq;
          const size_t o = (size_t)t * p.ldo + n0;
          if (vec && n0 + 3 < p.N) {
            const uint2 r = *reinterpret_cast<const uint2 *>(p.resid + o);
            const float rv[4] = {bf2f(r.x & 0xFFFFu), bf2f(r.x >> 16), bf2f(r.y & 0xFFFFu), bf2f(r.y >> 16)};
            float hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              hv[i] = bf2f(f2bf(acc[a][tt][i] * rs[tt] + rv[i]));
              sq += hv[i] * hv[i];
            }
            st_bf16x4(out + o, hv);
            if (p.out_pk) st_bf16x4(p.out_pk + frag_index(t, n0, p.out_pk_ntt), hv);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (n0 + i < p.N) {
                const uint16_t h = f2bf(acc[a][tt][i] * rs[tt] + bf2f(p.resid[o + i]));
                out[o + i] = h;
                if (p.out_pk) p.out_pk[frag_index(t, n0 + i, p.out_pk_ntt)] = h;
                const float f = bf2f(h);
                sq += f * f;
              }
            }
          }
        }
      }
      if (p.sq_out) {
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        if (gq == 0 && t < p.T) p.sq_out[(size_t)t * p.nblk + grp] = sq;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    uint16_t *out = static_cast<uint16_t *>(p.out);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = t0 + tt * 16 + l16;
      if (t >= p.T) continue;
      const int f0 = grp * 16 + 4 * gq;
      float hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = acc[0][tt][i] * rs[tt], u = acc[1][tt][i] * rs[tt];
        const float sig = 1.f / (1.f + __builtin_amdgcn_exp2f(-g * kLog2e));
        hv[i] = g * sig * u;
      }
      if (p.out_pk) {  // fragment layout only (the down projection's token operand)
        if (f0 + 3 < p.mat[0].rows) {
          st_bf16x4(p.out_pk + frag_index(t, f0, p.out_pk_ntt), hv);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (f0 + i < p.mat[0].rows) p.out_pk[frag_index(t, f0 + i, p.out_pk_ntt)] = f2bf(hv[i]);
        }
        continue;
      }
      uint16_t *o = out + (size_t)t * p.ldo + f0;
      if (vec && f0 + 3 < p.mat[0].rows) {
        st_bf16x4(o, hv);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (f0 + i < p.mat[0].rows) o[i] = f2bf(hv[i]);
      }
    }
  } else if constexpr (EPI == EPI_LOGITS) {
    float *out = static_cast<float *>(p.out);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = t0 + tt * 16 + l16;
      float v[8];
      float m = -INFINITY;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int n0 = grp * 32 + a * 16 + 4 * gq;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[a * 4 + i] = n0 + i < p.N ? acc[a][tt][i] * rs[tt] : -INFINITY;
          m = fmaxf(m, v[a * 4 + i]);
        }
        if (t < p.T) {
          float *o = out + (size_t)t * p.ldo + n0;
          if (vec && n0 + 3 < p.N) {
            *reinterpret_cast<float4 *>(o) = make_float4(v[a * 4], v[a * 4 + 1], v[a * 4 + 2], v[a * 4 + 3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (n0 + i < p.N) o[i] = v[a * 4 + i];
          }
        }
      }
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += __builtin_amdgcn_exp2f((v[e] - m) * kLog2e);
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (gq == 0 && t < p.T) {
        *reinterpret_cast<float2 *>(p.stats + ((size_t)t * p.nblk + grp) * 2) = make_float2(m, s);
      }
    }
  } else {  // EPI_QKV: tile 0 holds pair firsts i, tile 1 the partners i + hd/2
    const int gph = p.hd / 32;
    const int head = grp / gph, c = grp - head * gph;
    const int half = p.hd / 2;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int t = t0 + tt * 16 + l16;
      if (t >= p.T) continue;
      const int seq = p.tok_seq[t], pos = p.tok_pos[t];
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
          const float2 cs = *reinterpret_cast<const float2 *>(p.rope_cs + ((size_t)t * half + fi) * 2);
          ra[e] = a * cs.x - b * cs.y;
          rb[e] = b * cs.x + a * cs.y;
        } else {
          ra[e] = a;
          rb[e] = b;
        }
      }
      const int fi0 = 16 * c + 4 * gq;
      if (head >= p.hq && p.kvstage) {
        // int8 caches: stage the new key / value row; a later pass quantises it
        const int which = head < p.hq + p.hkv ? 0 : 1;
        const int kh = head - p.hq - which * p.hkv;
        uint16_t *st = p.kvstage + (((size_t)t * 2 + which) * p.hkv + kh) * p.hd;
        st_bf16x4(st + fi0, ra);
        st_bf16x4(st + fi0 + half, rb);
      } else if (head < p.hq) {
        uint16_t *q = p.qbuf + ((size_t)t * p.hq + head) * p.hd;
        st_bf16x4(q + fi0, ra);
        st_bf16x4(q + fi0 + half, rb);
      } else if (head < p.hq + p.hkv) {
        uint16_t *k = static_cast<uint16_t *>(p.kc[seq]) + ((size_t)(head - p.hq) * p.kv_cap + pos) * p.hd;
        st_bf16x4(k + fi0, ra);
        st_bf16x4(k + fi0 + half, rb);
      } else {
        // values in 32-position blocks: [n_kv][cap/32][hd][32]
        uint16_t *v = static_cast<uint16_t *>(p.vc[seq]) + (size_t)(head - p.hq - p.hkv) * p.hd * p.kv_cap +
                      (size_t)(pos >> 5) * p.hd * 32 + (pos & 31);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[(size_t)(fi0 + e) * 32] = f2bf(ra[e]);
          v[(size_t)(fi0 + half + e) * 32] = f2bf(rb[e]);
        }
      }
    }
  }
}

// Waves per workgroup for KW waves per unit.
template <int KW> constexpr int waves_per_wg() { return KW > 4 ? KW : 4; }

// K split across workgroups: store this unit's partial tile with device-scope
// stores, count its arrival, and if it is the last of the splits, add all
// partials in split order into acc (bitwise repeatable).  Returns whether this
// unit is the last (and must run the epilogue).
template <int TT>
__device__ __forceinline__ bool split_reduce(const GemmParams &p, floatx4 (&acc)[2][TT], int grp, int tb, int split,
                                             int lane) {
  constexpr int TILE = 2 * TT * 4 * 64;  // one partial value per (tile, token tile, row, lane)
  const size_t tile_id = (size_t)tb * p.nblk + grp;
  float *mine = p.partial + ((size_t)split * p.nblk * p.ntblk + tile_id) * TILE;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) store_dev(mine + ((a * TT + tt) * 4 + i) * 64 + lane, acc[a][tt][i]);
  wait_vmem();
  int old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(p.counters + tile_id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old != p.splits - 1) return false;
  if (lane == 0) __hip_atomic_store(p.counters + tile_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[a][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < p.splits; ++sp) {
    const float *src = p.partial + ((size_t)sp * p.nblk * p.ntblk + tile_id) * TILE;
    // half a tile is loaded before any of it is added, so that its loads are
    // in flight together
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      float v[TT][4];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[tt][i] = load_dev(src + ((a * TT + tt) * 4 + i) * 64 + lane);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[a][tt][i] += v[tt][i];
    }
  }
  return true;
}

// G = K steps of weights and tokens in flight per wave: 2 for long streams
// (many resident waves share the work), 4 or 8 for short ones (one or two
// rounds of loads per wave).  The one-wave-per-unit bf16 stream (the LM head
// at up to 32 tokens) is held to 6 resident workgroups per CU (80 registers):
// a few registers more drop it to 5 and cost 2% of its time; forcing 8 (64
// registers) spills and measured slower.
// KW = waves per unit: the unit's K range is cut into KW consecutive pieces,
// one per wave of the same workgroup, and the pieces are added through LDS in
// wave order (bitwise repeatable) before the epilogue, which the unit's first
// wave runs.  This fills the chip for short row counts without sending
// partial sums through memory.
template <int WT, int TT, int EPI, int G, int KW> constexpr int min_wg_per_cu() {
  return (KW == 1 && WT == WT_BF16 && EPI == EPI_LOGITS && TT <= 2 && G <= 2) ? 6 : 1;
}


template <int WT, int TT, int EPI, int G, int KW>
__global__ __launch_bounds__(64 * waves_per_wg<KW>(), (min_wg_per_cu<WT, TT, EPI, G, KW>())) void gemm_kernel(
    GemmParams p) {
  constexpr int WV = waves_per_wg<KW>();
  constexpr int UPW = WV / KW;  // units per workgroup
  constexpr int NACC = 2 * TT * 4;
  // gate||up with several waves per unit: the token block's rows of partial
  // sums of squares ([T][nparts], from the previous projection) are copied
  // straight into LDS when the workgroup starts, so the epilogue forms the
  // RMSNorm scales from LDS instead of a scattered global round trip at the end
  constexpr bool kRsl = EPI == EPI_SWIGLU && KW > 1 && TT <= 2;
  constexpr int kRslI = kRsl ? (TT * 16 * kRsPartsMax / 4 + 64 * WV - 1) / (64 * WV) : 1;
  __shared__ float kred[KW > 1 ? WV * NACC * 64 : 1];
  __shared__ __align__(16) unsigned char xl[KW == 1 ? xl_bytes<WT, TT, G>() : 16];
  __shared__ __align__(16) float rsl[kRsl ? kRslI * WV * 64 * 4 : 4];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = wave % KW, slot = wave / KW;
  const int gq = lane >> 4, l16 = lane & 15;
  // KW == 1 keeps the dispatch order (measured faster for the long streams);
  // split launches run a unit's neighbours on one XCD
  const int wg = KW == 1 ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  const int ngrp = p.nblk;
  int tb, grp, split;
  bool active;
  if constexpr (KW == 1) {
    // the workgroup's units are UPW consecutive row groups of one token block
    // and K split, so they share the token operand; token block fastest, so
    // the workgroups that need the same weights run at the same time
    const int nq = (ngrp + UPW - 1) / UPW;
    tb = wg % p.ntblk;
    const int rest = wg / p.ntblk;
    split = rest / nq;
    grp = (rest % nq) * UPW + slot;
    active = grp < ngrp;
    grp = min(grp, ngrp - 1);  // idle waves still load their share of the tokens
  } else {
    const int nunits = ngrp * p.splits * p.ntblk;
    active = wg < nunits;
    const int unit = min(wg, nunits - 1);
    tb = unit % p.ntblk;
    const int rest = unit / p.ntblk;
    grp = rest % ngrp;
    split = rest / ngrp;
  }
  const int t0 = tb * TT * 16;
  const int u0 = (int)((long long)split * p.ksteps / p.splits);
  const int u1 = (int)((long long)(split + 1) * p.ksteps / p.splits);
  // this wave's piece of the unit's K range (all of it when KW == 1)
  const int s0 = u0 + (u1 - u0) * sub / KW;
  const int nsteps = (active || KW == 1) ? u0 + (u1 - u0) * (sub + 1) / KW - s0 : 0;

  // weight stream of each of the unit's two tiles (rows past the end of a
  // matrix stream its first tile; their results are dropped)
  WSrc<WT> src[2];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    int mi = 0, pr0 = 0;
    if (!map_row(p, grp, tile, 0, mi, pr0)) { mi = 0; pr0 = 0; }
    int pr = pr0 + l16;
    if (pr >= p.mat[mi].rows) pr = pr0;
    src[tile] = make_src<WT>(p.mat[mi], pr, pr0, p.K, p.ksteps, p.packed, lane, gq);
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
  float ssq[TT];  // rms_inline: this lane's share of its tokens' sums of squares
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) ssq[tt] = 0.f;

  bool rs_lds = false;
  if constexpr (kRsl) {
    // row tok of the block (token min(t0 + tok, T - 1)) at rsl[tok * nparts];
    // 16-byte pieces in lane order, every lane loading (past the rows' end it
    // repeats the last piece into space nobody reads); without partial sums
    // the loads read the token operand and the result is unused
    rs_lds = p.rparts && !p.rnorm && (p.nparts & 3) == 0 && p.nparts > 0 && p.nparts <= kRsPartsMax;
    const int q4 = rs_lds ? p.nparts >> 2 : 1;
    const int nch = TT * 16 * q4;
#pragma unroll
    for (int i = 0; i < kRslI; ++i) {
      const int cb = (i * WV + wave) * 64;
      const int c = min(cb + lane, nch - 1);
      const int tok = c / q4, q = c - tok * q4;
      const void *src = rs_lds ? static_cast<const void *>(p.rparts + (size_t)min(t0 + tok, p.T - 1) * p.nparts + 4 * q)
                               : static_cast<const void *>(p.x);
      load_lds16(src, rsl + cb * 4);
    }
  }

  // Grouped prefetch: G steps of weights and tokens in flight per wave, then
  // compute.  A shallow group keeps the register count low, so many waves are
  // resident and together keep the memory system busy.
  if constexpr (KW == 1) {
    // token operand through LDS: each step's fragments are loaded once per
    // workgroup (fragment f by wave f % WV, straight into LDS in lane order)
    // and read by every unit; a ring of two groups lets the loads of group
    // i + 1 start while slower waves still read group i
    constexpr int NXF = xfrags<WT>();
    constexpr int XF = TT * NXF;
    constexpr int NL = (XF + WV - 1) / WV;  // fragments loaded per wave and step
    constexpr int SLOT = G * XF * 1024;
    constexpr int KS = kstep<WT>();
    const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform, in a scalar register
    const uint16_t *xa[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int f = min(wv + WV * i, XF - 1);
      const int tt = f / NXF, m = f - tt * NXF;
      xa[i] = p.x + (size_t)min(t0 + tt * 16 + l16, p.T - 1) * p.K + xoff<WT>(m, gq);
    }
    for (int base = 0, gi = 0; base < nsteps; base += G, ++gi) {
      unsigned char *xs = xl + (gi & 1) * SLOT;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int st = s0 + min(base + j, nsteps - 1);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int f = wv + WV * i;
          if (f < XF)
            load_lds16(xa[i] + st * KS, xs + (j * XF + f) * 1024);
        }
      }
      WStep<WT> wbuf[G][2];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int st = s0 + min(base + j, nsteps - 1);
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) wbuf[j][tile] = load_w<WT>(src[tile], st);
      }
      wait_vmem();
      __syncthreads();
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (base + j < nsteps) {
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            XStep<WT> xv;
#pragma unroll
            for (int m = 0; m < NXF; ++m) xv.v[m] = ld_v4(xs + ((j * XF + tt * NXF + m) * 64 + lane) * 16);
            if (p.rms_inline) {
#pragma unroll
              for (int m = 0; m < NXF; ++m) {
                const uint32_t w4[4] = {xv.v[m].x, xv.v[m].y, xv.v[m].z, xv.v[m].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float lo = __uint_as_float(w4[e] << 16), hi = __uint_as_float(w4[e] & 0xFFFF0000u);
                  ssq[tt] += lo * lo + hi * hi;
                }
              }
            }
            mma_tile<WT>(wbuf[j][0], xv, acc[0][tt]);
            mma_tile<WT>(wbuf[j][1], xv, acc[1][tt]);
          }
        }
      }
    }
    if (!active) return;
  } else {
    // bf16 token fragments: row-major rows (sixteen 64-byte pieces per load) or
    // the fragment layout (one contiguous KiB); both affine in the step
    const uint16_t *xb[TT];
    int xstride = 64, xoff1 = 32;
    if constexpr (WT == WT_BF16) {
      if (p.xp) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) xb[tt] = p.xp + (size_t)(tb * TT + tt) * 1024 + lane * 8;
        xstride = p.xp_ntt * 1024;
        xoff1 = 512;
      } else {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) xb[tt] = xr[tt] + 8 * gq;
      }
    }
    for (int base = 0; base < nsteps; base += G) {
      WStep<WT> wbuf[G][2];
      XStep<WT> xbuf[G][TT];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int st = s0 + min(base + j, nsteps - 1);
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) wbuf[j][tile] = load_w<WT>(src[tile], st);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          if constexpr (WT == WT_BF16) {
            const uint16_t *b = xb[tt] + (size_t)st * xstride;
            xbuf[j][tt].v[0] = *reinterpret_cast<const uint4 *>(b);
            xbuf[j][tt].v[1] = *reinterpret_cast<const uint4 *>(b + xoff1);
          } else {
            xbuf[j][tt] = load_x<WT>(xr[tt], st, gq);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        if (base + j < nsteps) {
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            mma_tile<WT>(wbuf[j][0], xbuf[j][tt], acc[0][tt]);
            mma_tile<WT>(wbuf[j][1], xbuf[j][tt], acc[1][tt]);
          }
        }
      }
    }
  }

  // ---- in-workgroup reduction of the unit's K pieces ------------------------
  if constexpr (KW > 1) {
    if constexpr (kRsl) wait_vmem();  // this wave's copies into rsl (the barrier publishes them)
    if (sub != 0) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) kred[(wave * NACC + (a * TT + tt) * 4 + i) * 64 + lane] = acc[a][tt][i];
    }
    __syncthreads();
    if (!active || sub != 0) return;
#pragma unroll 1
    for (int w = 1; w < KW; ++w) {
      const float *r = kred + (size_t)(wave + w) * NACC * 64 + lane;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[a][tt][i] += r[((a * TT + tt) * 4 + i) * 64];
    }
  }

  // ---- K-split reduction across units ---------------------------------------
  if (p.splits > 1 && !split_reduce<TT>(p, acc, grp, tb, split, lane)) return;

  if (KW == 1 && p.rms_inline) {
    // every lane group gq read a quarter of each token's K values
    float rs[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      float sq = ssq[tt];
      sq += __shfl_xor(sq, 16);
      sq += __shfl_xor(sq, 32);
      rs[tt] = 1.f / sqrtf(sq / static_cast<float>(p.K) + p.eps);
    }
    epilogue_rs<TT, EPI>(p, acc, grp, t0, gq, l16, rs);
  } else if (kRsl && rs_lds) {
    // the same partial sums in the same order as token_scales, from LDS
    float rs[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int tok = min(t0 + tt * 16 + l16, p.T - 1) - t0;
      const float *pr = rsl + tok * p.nparts;
      float s = 0.f;
#pragma unroll 8
      for (int g = gq; g < p.nparts; g += 4) s += pr[g];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      rs[tt] = 1.f / sqrtf(s / static_cast<float>(p.K) + p.eps);
    }
    epilogue_rs<TT, EPI>(p, acc, grp, t0, gq, l16, rs);
  } else {
    epilogue<TT, EPI>(p, acc, grp, t0, gq, l16);
  }
}

// ---------------------------------------------------------------------------
// LDS-tiled GEMM for many stacked tokens (bf16, packed weights).
//
// With hundreds of tokens the per-wave streaming kernel above is bound by
// each wave fetching its own copy of the token operand.  Here a workgroup of
// 8 waves computes 8 row groups (256 weight rows) x 128 tokens: each K step
// (64) of the weight fragments (in their packed, lane-ordered form) and of the
// token rows is loaded straight into LDS (global_load_lds, 16 bytes per lane)
// and read by every wave; each wave computes 2 row groups x 64 tokens (32
// MFMAs per step).  Three LDS buffers keep the loads of the next two steps in
// flight during the current step's MFMAs.  A token row's eight 16-byte chunks
// are stored XOR-swizzled by the row index, which spreads the MFMA operand
// reads over the LDS banks.  Workgroups run token block fastest (XCD-aware),
// so the token blocks of one row block share its weights in L2.
constexpr int kTThreads = 512;
constexpr int kTGroups = 8;                                  // 32-row groups per workgroup
constexpr int kTTok = 128;                                   // tokens per workgroup
constexpr int kTWBytes = kTGroups * 2 * 2 * 64 * 16;         // 16 tiles x 2 halves x 64 lanes x 16 B
constexpr int kTXBytes = kTTok * 128;                        // 128 rows x 64 bf16
constexpr int kTBuf = kTWBytes + kTXBytes;
constexpr int kTStages = 3;
constexpr int kTLds = kTStages * kTBuf;
constexpr int kTWPer = kTWBytes / 16 / kTThreads;            // weight fragments loaded per thread (4)
constexpr int kTXPer = kTXBytes / 16 / kTThreads;            // token chunks loaded per thread (2)

// Workgroup barrier for the LDS ring: __syncthreads() would also wait for all
// of this wave's outstanding global loads (its release fence covers the
// direct-to-LDS loads), draining the prefetch.  The waits it needs are issued
// explicitly (vmcnt for this wave's loads of the step); the empty asm keeps the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// LDS byte pointers and 16-byte reads through them (address space 3).
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
__device__ __forceinline__ uint4 ld_lds_v4(const lds_u8 *p) {
  return __builtin_bit_cast(uint4, *reinterpret_cast<lds_u32x4 *>(p));
}

template <int EPI>
__global__ __launch_bounds__(kTThreads, 1) void gemm_tiled_kernel(GemmParams p) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, l16 = lane & 15;
  const int ntb = (p.T + kTTok - 1) / kTTok;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int tb = wg % ntb, rb = wg / ntb;
  const int gp = wave & 3, th = wave >> 2;  // groups 2gp, 2gp+1 of the block; tokens th*64 ..

  // Load j of this thread fills LDS bytes [16 f, 16 f + 16) of its region,
  // f = tid + 512 j (a wave's 64 lanes fill one contiguous KiB).
  //  weights: fragment f = (tile f/128, half (f/64)%2, lane f%64) of the packed layout
  //  tokens:  row f/8, slot f%8 holding chunk (f%8) ^ (row%8) of the row's 64 values
  const unsigned char *wsrc[kTWPer];
  size_t wstep[kTWPer];   // bytes between K steps of the fragment's matrix (step-major)
  uint32_t xoff[kTXPer];  // element offsets of this thread's token chunks (step 0)
#pragma unroll
  for (int j = 0; j < kTWPer; ++j) {
    const int f = tid + kTThreads * j;
    const int q = f >> 7, m = (f >> 6) & 1, fl = f & 63;
    int mi = 0, pr0 = 0;
    if (!map_row(p, rb * kTGroups + (q >> 1), q & 1, 0, mi, pr0)) {
      mi = 0;
      pr0 = 0;
    }
    const size_t g = (size_t)(pr0 / 32);
    const int a = (pr0 / 16) & 1;
    wsrc[j] = static_cast<const unsigned char *>(p.mat[mi].w) + (((g * 2 + a) * 2 + m) * 64 + fl) * 16;
    wstep[j] = (size_t)((p.mat[mi].rows + 31) / 32) * 4096;
  }
#pragma unroll
  for (int j = 0; j < kTXPer; ++j) {
    const int f = tid + kTThreads * j;
    const int r = f >> 3, c = (f & 7) ^ (r & 7);
    xoff[j] = (uint32_t)min(tb * kTTok + r, p.T - 1) * (uint32_t)p.K + c * 8;
  }
  // wave-uniform LDS destination of load j (lane offsets are implicit)
  const int wbase = wave * 64 * 16;

  floatx4 acc[2][2][4];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[gi][a][tt] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int st, int buf) {
    unsigned char *b = lds + buf * kTBuf;
#pragma unroll
    for (int j = 0; j < kTWPer; ++j)
      load_lds16(wsrc[j] + (size_t)st * wstep[j], b + wbase + j * kTThreads * 16);
#pragma unroll
    for (int j = 0; j < kTXPer; ++j)
      load_lds16(p.x + xoff[j] + st * 64, b + kTWBytes + wbase + j * kTThreads * 16);
  };

  const int ns = p.ksteps;
  issue(0, 0);
  if (ns > 1) issue(1, 1);
  for (int st = 0; st < ns; ++st) {
    // this wave's loads of step st are done once at most the next step's remain
    if (st + 1 < ns)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (kTWPer + kTXPer));  // vmcnt(6)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0)
    ring_barrier();  // everyone's step st is in LDS; everyone is done with step st - 1
    if (st + 2 < ns) issue(st + 2, (st + 2) % kTStages);
    const unsigned char *bw = lds + (st % kTStages) * kTBuf;
    const unsigned char *bx = bw + kTWBytes;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bf16x8 wv[2][2];
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int a = 0; a < 2; ++a)
          wv[gi][a] = as_bf16x8(*reinterpret_cast<const uint4 *>(
              bw + ((((2 * gp + gi) * 2 + a) * 2 + m) * 64 + lane) * 16));
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int r = th * 64 + tt * 16 + l16;
        const bf16x8 xv = as_bf16x8(*reinterpret_cast<const uint4 *>(
            bx + r * 128 + (((4 * m + gq) ^ (r & 7)) * 16)));
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
          for (int a = 0; a < 2; ++a) acc[gi][a][tt] = mfma16x16x32(wv[gi][a], xv, acc[gi][a][tt]);
      }
    }
  }

#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int grp = rb * kTGroups + 2 * gp + gi;
    if (grp < p.nblk) epilogue<4, EPI>(p, acc[gi], grp, tb * kTTok + th * 64, gq, l16);
  }
}

// Grid of the tiled kernel: row blocks x token blocks.
inline int tiled_grid(const GemmParams &p) {
  return ((p.nblk + kTGroups - 1) / kTGroups) * ((p.T + kTTok - 1) / kTTok);
}

template <int EPI>
hipError_t launch_tiled_epi(const GemmParams &p, hipStream_t s, int trace_class) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_tiled_kernel<EPI>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kTLds);
    attr = true;
  }
  trace_before(trace_class, s);
  hipLaunchKernelGGL((gemm_tiled_kernel<EPI>), dim3(tiled_grid(p)), dim3(kTThreads), kTLds, s, p);
  trace_after(trace_class, s);
  return hipGetLastError();
}

inline hipError_t launch_tiled(const GemmParams &p, hipStream_t s, int trace_class) {
  switch (p.epi) {
    case EPI_QKV: return launch_tiled_epi<EPI_QKV>(p, s, trace_class);
    case EPI_RESID: return launch_tiled_epi<EPI_RESID>(p, s, trace_class);
    case EPI_SWIGLU: return launch_tiled_epi<EPI_SWIGLU>(p, s, trace_class);
    default: return launch_tiled_epi<EPI_LOGITS>(p, s, trace_class);
  }
}

// ---------------------------------------------------------------------------
// Wide streaming GEMM for many stacked tokens (bf16, packed weights).
//
// A workgroup of 4 waves computes 8 row groups (256 weight rows) x 16 TT
// tokens over a K range.  Each wave owns two row groups (64 rows) and streams
// their weight fragments straight from HBM into registers; the token operand
// of a step is loaded once per workgroup straight into LDS (fragment order)
// and read by all four waves.  Both run D steps ahead of the MFMAs (a ring of
// D + 1 register buffers and D + 1 LDS slots): a step's MFMAs take well under
// an HBM round trip, so one step of lookahead leaves every step waiting for
// its weights.  Per step a wave issues 16 TT MFMAs for 2 TT 16-byte LDS reads
// (256 B of LDS per MFMA), half of what staging the weights through LDS as
// well would read.  K splits across workgroups go through the same
// deterministic last-arriver reduction as the streaming kernel, and the
// epilogues are the same.
constexpr int kWGroups = 8;  // 32-row groups per workgroup (two per wave)

// f(std::integral_constant<int, k>()) for k = 0 .. N-1 (compile-time indices
// keep register ring slots static)
template <class F, int... K>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>()), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>());
}


template <int EPI, int TT, int D>
__global__ __launch_bounds__(256, (D <= 2 && TT <= 4 ? 2 : 1)) void gemm_wide_kernel(GemmParams p) {
  constexpr int NB = D + 1;   // ring slots (registers and LDS)
  constexpr int XF = TT * 2;  // token fragments (1 KiB) per step
  constexpr int XW = XF / 4;  // loaded by each wave
  constexpr int PER = 8 + XW; // loads a wave issues per step (weights, tokens)
  constexpr int SLOT = XF * 1024;
  static_assert(XF % 4 == 0, "token fragments must split over the four waves");
  static_assert((D - 1) * PER <= 63, "outstanding loads beyond the vmcnt range");
  static_assert(NB <= 5 && NB * SLOT <= 160 * 1024, "ring slots");
  // one LDS object per ring slot: reads of one slot then provably do not
  // alias the direct-to-LDS loads in flight into the others, and the compiler
  // does not wait for those loads before every LDS read
  __shared__ __align__(16) unsigned char xr0[SLOT], xr1[SLOT], xr2[SLOT];
  __shared__ __align__(16) unsigned char xr3[NB > 3 ? SLOT : 16], xr4[NB > 4 ? SLOT : 16];
  auto slot_of = [&](auto kc) -> lds_u8 * {
    constexpr int k = decltype(kc)::value;
    if constexpr (k == 0) return (lds_u8 *)xr0;
    else if constexpr (k == 1) return (lds_u8 *)xr1;
    else if constexpr (k == 2) return (lds_u8 *)xr2;
    else if constexpr (k == 3) return (lds_u8 *)xr3;
    else return (lds_u8 *)xr4;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gq = lane >> 4, l16 = lane & 15;
  const int nrb = (p.nblk + kWGroups - 1) / kWGroups;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  // token block fastest: the workgroups that read a row block's weights run
  // side by side on one XCD and find them in its L2
  const int tb = wg % p.ntblk;
  const int rest = wg / p.ntblk;
  const int rb = rest % nrb, split = rest / nrb;
  const int t0 = tb * TT * 16;
  const int u0 = (int)((long long)split * p.ksteps / p.splits);
  const int u1 = (int)((long long)(split + 1) * p.ksteps / p.splits);
  const int ns = u1 - u0;

  int grp[2];
  bool gact[2];
  WSrc<WT_BF16> src[2][2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int gr = rb * kWGroups + 2 * wave + gi;
    gact[gi] = gr < p.nblk;
    grp[gi] = min(gr, p.nblk - 1);  // idle groups stream a valid group; results dropped
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      int mi = 0, pr0 = 0;
      if (!map_row(p, grp[gi], a, 0, mi, pr0)) { mi = 0; pr0 = 0; }
      src[gi][a] = make_src<WT_BF16>(p.mat[mi], pr0, pr0, p.K, p.ksteps, 1, lane, gq);
    }
  }
  // token fragments this wave loads: f = wave + 4 i -> (tt = f / 2, half m = f % 2),
  // as element offsets from the split's first step
  const uint16_t *xbase = p.x + (size_t)u0 * 64;
  uint32_t xo[XW];
#pragma unroll
  for (int i = 0; i < XW; ++i) {
    const int f = wave + 4 * i, tt = f >> 1, m = f & 1;
    xo[i] = (uint32_t)min(t0 + tt * 16 + l16, p.T - 1) * (uint32_t)p.K + 32 * m + 8 * gq;
  }

  floatx4 acc[2][2][TT];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[gi][a][tt] = floatx4{0.f, 0.f, 0.f, 0.f};

  WStep<WT_BF16> wb[NB][2][2];  // [slot][group][tile]
  // Step st's tokens go to LDS slot st % NB and its weights to wb[st % NB].
  // The loop is branch-free so the compiler can count which loads feed which
  // registers (behind conditional loads it drains every load at each step):
  // steps past the end reload the last step (clamped addresses) and skip
  // their MFMAs (a wave-uniform branch around compute only).
  auto issue = [&](int st, auto kc, lds_u8 *slot) {
    constexpr int k = decltype(kc)::value;
    const int sc = min(st, ns - 1);
#pragma unroll
    for (int i = 0; i < XW; ++i) load_lds16(xbase + xo[i] + sc * 64, (lds_void *)(slot + (wave + 4 * i) * 1024));
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int a = 0; a < 2; ++a) wb[k][gi][a] = load_w<WT_BF16>(src[gi][a], u0 + sc);
  };
  if (ns > 0) {
    // steps in order: the waits count loads in issue order
    static_for<D>([&](auto kc) {
      issue(decltype(kc)::value, kc, slot_of(kc));
      __builtin_amdgcn_sched_barrier(0);
    });
    // step st (slot b = st % NB): wait for this wave's loads of step st (the
    // D - 1 later steps' stay in flight) and its LDS reads of step st - 1,
    // barrier, compute, then issue step st + D into the slot step st - 1
    // used.  The barrier is the bare instruction (the compiler's scheduler
    // keeps memory accesses on their side of it); a memory clobber there, as
    // in the other kernels' ring_barrier, pins the schedule of the whole step
    // to source order, and each LDS read then waits before its MFMAs.
    auto step = [&](int st, auto bc) {
      constexpr int b = decltype(bc)::value;
      constexpr int later = (D - 1) * PER;
      __builtin_amdgcn_s_waitcnt(0x0070 | (later & 15) | ((later >> 4) << 14));  // vmcnt(later) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();  // step st's tokens in LDS for everyone; everyone is done with step st - 1
      if (st < ns) {
        const lds_u8 *xs = slot_of(bc);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            const bf16x8 xv = as_bf16x8(ld_lds_v4(xs + ((tt * 2 + m) * 64 + lane) * 16));
#pragma unroll
            for (int gi = 0; gi < 2; ++gi)
#pragma unroll
              for (int a = 0; a < 2; ++a)
                acc[gi][a][tt] = mfma16x16x32(as_bf16x8(wb[b][gi][a].v[m]), xv, acc[gi][a][tt]);
          }
        // batches of four fragments: a batch's four reads are issued after
        // the first four of the previous batch's 16 MFMAs, so the wait before
        // a batch (the compiler waits for every outstanding LDS read) comes
        // 12 MFMAs after them
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
#pragma unroll
        for (int i = 0; i < 2 * TT / 4 - 1; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // DS read
          __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);  // MFMA
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      }
      constexpr int nb = (b + D) % NB;
      issue(st + D, std::integral_constant<int, nb>(), slot_of(std::integral_constant<int, nb>()));
    };
    for (int st0 = 0; st0 < ns; st0 += NB) static_for<NB>([&](auto kc) { step(st0 + decltype(kc)::value, kc); });
    wait_vmem();  // the clamped tail loads
  }

#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    if (!gact[gi]) continue;
    if (p.splits > 1 && !split_reduce<TT>(p, acc[gi], grp[gi], tb, split, lane)) continue;
    epilogue<TT, EPI>(p, acc[gi], grp[gi], t0, gq, l16);
  }
}

// Grid of the wide kernel: row blocks x token blocks x K splits.
inline int wide_grid(const GemmParams &p) {
  return ((p.nblk + kWGroups - 1) / kWGroups) * p.ntblk * p.splits;
}

template <int EPI, int TT, int D>
hipError_t launch_wide_d(const GemmParams &p, hipStream_t s, int trace_class) {
  trace_before(trace_class, s);
  hipLaunchKernelGGL((gemm_wide_kernel<EPI, TT, D>), dim3(wide_grid(p)), dim3(256), 0, s, p);
  trace_after(trace_class, s);
  return hipGetLastError();
}

// The wide streaming kernel for packed int4 weights: the same tiling (8 row
// groups x 16 TT tokens per workgroup, each wave streaming two row groups'
// codes and scales into registers, the token operand shared in LDS), with
// int4 steps of 128 along K.  Each step's weights are converted to bf16 once
// in registers (dequant8) and reused for every token tile, so a weight is
// read and converted once per 16 TT tokens (the int4 streaming kernel does so
// per 16 x up to 4 tokens).  The token fragments follow the int4 operand
// order (lane group gq holds one group of 32 along K).  D = 2 steps of
// lookahead (an LDS ring of three slots of TT x 4 KiB; a step is 128 of K).
template <int EPI, int TT, int D>
__global__ __launch_bounds__(256, (TT >= 8 ? 1 : 2)) void gemm_wide4_kernel(GemmParams p) {
  constexpr int NB = D + 1;   // ring slots (registers and LDS)
  constexpr int XF = TT * 4;  // token fragments (1 KiB) per step
  constexpr int XW = XF / 4;  // loaded by each wave
  constexpr int PER = 8 + XW; // loads a wave issues per step (4 x codes and scales, tokens)
  constexpr int SLOT = XF * 1024;
  static_assert(NB == 3, "three ring slots");
  static_assert((D - 1) * PER <= 63, "outstanding loads beyond the vmcnt range");
  __shared__ __align__(16) unsigned char xr0[SLOT], xr1[SLOT], xr2[SLOT];
  auto slot_of = [&](auto kc) -> unsigned char * {
    constexpr int k = decltype(kc)::value;
    if constexpr (k == 0) return xr0;
    else if constexpr (k == 1) return xr1;
    else return xr2;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gq = lane >> 4, l16 = lane & 15;
  const int nrb = (p.nblk + kWGroups - 1) / kWGroups;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int tb = wg % p.ntblk;
  const int rest = wg / p.ntblk;
  const int rb = rest % nrb, split = rest / nrb;
  const int t0 = tb * TT * 16;
  const int u0 = (int)((long long)split * p.ksteps / p.splits);
  const int u1 = (int)((long long)(split + 1) * p.ksteps / p.splits);
  const int ns = u1 - u0;

  int grp[2];
  bool gact[2];
  WSrc<WT_INT4> src[2][2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int gr = rb * kWGroups + 2 * wave + gi;
    gact[gi] = gr < p.nblk;
    grp[gi] = min(gr, p.nblk - 1);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      int mi = 0, pr0 = 0;
      if (!map_row(p, grp[gi], a, 0, mi, pr0)) { mi = 0; pr0 = 0; }
      src[gi][a] = make_src<WT_INT4>(p.mat[mi], pr0, pr0, p.K, p.ksteps, 1, lane, gq);
    }
  }
  // token fragments this wave loads: f = wave + 4 i -> (tt = f / 4, m = f % 4),
  // lane (gq, l16) holding x[token][128 s + 32 gq + 8 m .. + 7]
  const uint16_t *xa[XW];
#pragma unroll
  for (int i = 0; i < XW; ++i) {
    const int f = wave + 4 * i, tt = f >> 2, m = f & 3;
    xa[i] = p.x + (size_t)min(t0 + tt * 16 + l16, p.T - 1) * p.K + (size_t)u0 * 128 + 32 * gq + 8 * m;
  }

  floatx4 acc[2][2][TT];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[gi][a][tt] = floatx4{0.f, 0.f, 0.f, 0.f};

  WStep<WT_INT4> wb[NB][2][2];  // [slot][group][tile]
  // branch-free as the bf16 kernel: steps past the end reload the last one
  // (and convert it with scale 0)
  auto issue = [&](int st, auto kc) {
    constexpr int k = decltype(kc)::value;
    const int sc = min(st, ns - 1);
    unsigned char *slot = slot_of(kc);
#pragma unroll
    for (int i = 0; i < XW; ++i) load_lds16(xa[i] + sc * 128, slot + (wave + 4 * i) * 1024);
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int a = 0; a < 2; ++a) wb[k][gi][a] = load_w<WT_INT4>(src[gi][a], u0 + sc);
  };
  // fragment m (K 32 gq + 8 m of the step) of the four tiles of ring slot k, in bf16
  auto convert = [&](auto kc, auto mc, bool live, bf16x8 (&out)[2][2]) {
    constexpr int k = decltype(kc)::value, m = decltype(mc)::value;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const uint4 &v = wb[k][gi][a].v;
        const uint32_t word = m == 0 ? v.x : m == 1 ? v.y : m == 2 ? v.z : v.w;
        out[gi][a] = dequant8(word, live ? bf2f(static_cast<uint16_t>(wb[k][gi][a].s)) : 0.f);
      }
  };
  // Each step runs in four phases, one per fragment m: the MFMAs of phase m
  // (4 tiles x TT token tiles) are interleaved with the conversion of
  // fragment m + 1 and the LDS reads of its token fragments (phase 3 converts
  // fragment 0 of the next step), so the VALU work of the conversion hides
  // under the matrix pipe.
  bf16x8 wv[2][2][2];  // [phase parity][group][tile]
  bf16x8 xv[2][TT];    // [phase parity][token tile]
  if (ns > 0) {
    // steps in order: the waits count loads in issue order
    static_for<D>([&](auto kc) {
      issue(decltype(kc)::value, kc);
      __builtin_amdgcn_sched_barrier(0);
    });
    convert(std::integral_constant<int, 0>(), std::integral_constant<int, 0>(), true, wv[0]);
    auto step = [&](int st, auto bc) {
      constexpr int b = decltype(bc)::value;
      constexpr int later = (D - 1) * PER;
      __builtin_amdgcn_s_waitcnt(0x0F70 | (later & 15) | ((later >> 4) << 14));
      ring_barrier();  // step st's tokens in LDS for everyone; everyone is done with step st - 1
      // keep every instruction of this step below the wait: hoisting the
      // conversion of a later step's weights above it makes the compiler
      // drain all loads in flight
      __builtin_amdgcn_sched_barrier(0);
      issue(st + D, std::integral_constant<int, (b + D) % NB>());
      const unsigned char *xs = slot_of(bc);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) xv[0][tt] = as_bf16x8(ld_v4(xs + ((tt * 4) * 64 + lane) * 16));
      __builtin_amdgcn_sched_barrier(0);
      const bool live = st < ns, live_next = st + 1 < ns;
      static_for<4>([&](auto mc) {
        constexpr int m = decltype(mc)::value, P = m & 1;
        if constexpr (m < 3) {
          convert(bc, std::integral_constant<int, m + 1>(), live, wv[P ^ 1]);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
            xv[P ^ 1][tt] = as_bf16x8(ld_v4(xs + ((tt * 4 + m + 1) * 64 + lane) * 16));
        } else {
          // the next step's loads (all but this step's issue) have landed
          __builtin_amdgcn_s_waitcnt(0x0F70 | (PER & 15) | ((PER >> 4) << 14));
          __builtin_amdgcn_sched_barrier(0);
          convert(std::integral_constant<int, (b + 1) % NB>(), std::integral_constant<int, 0>(), live_next, wv[0]);
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int a = 0; a < 2; ++a) acc[gi][a][tt] = mfma16x16x32(wv[P][gi][a], xv[P][tt], acc[gi][a][tt]);
        // one MFMA, then the next phase's LDS reads and conversion in the gaps
#pragma unroll
        for (int i = 0; i < 4 * TT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          if (i < TT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    for (int st0 = 0; st0 < ns; st0 += NB) static_for<NB>([&](auto kc) { step(st0 + decltype(kc)::value, kc); });
    wait_vmem();  // the clamped tail loads
  }

#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    if (!gact[gi]) continue;
    if (p.splits > 1 && !split_reduce<TT>(p, acc[gi], grp[gi], tb, split, lane)) continue;
    epilogue<TT, EPI>(p, acc[gi], grp[gi], t0, gq, l16);
  }
}

template <int EPI, int TT>
hipError_t launch_wide4_tt(const GemmParams &p, hipStream_t s, int trace_class) {
  trace_before(trace_class, s);
  hipLaunchKernelGGL((gemm_wide4_kernel<EPI, TT, 2>), dim3(wide_grid(p)), dim3(256), 0, s, p);
  trace_after(trace_class, s);
  return hipGetLastError();
}

// tok_tiles: 16-token tiles per block (1, 2, 4 or 8)
template <int EPI>
hipError_t launch_wide4_epi(const GemmParams &p, int tok_tiles, hipStream_t s, int trace_class) {
  switch (tok_tiles) {
    case 1: return launch_wide4_tt<EPI, 1>(p, s, trace_class);
    case 2: return launch_wide4_tt<EPI, 2>(p, s, trace_class);
    case 4: return launch_wide4_tt<EPI, 4>(p, s, trace_class);
    default: return launch_wide4_tt<EPI, 8>(p, s, trace_class);
  }
}

inline hipError_t launch_wide4(const GemmParams &p, int tok_tiles, hipStream_t s, int trace_class) {
  switch (p.epi) {
    case EPI_QKV: return launch_wide4_epi<EPI_QKV>(p, tok_tiles, s, trace_class);
    case EPI_RESID: return launch_wide4_epi<EPI_RESID>(p, tok_tiles, s, trace_class);
    case EPI_SWIGLU: return launch_wide4_epi<EPI_SWIGLU>(p, tok_tiles, s, trace_class);
    default: return launch_wide4_epi<EPI_LOGITS>(p, tok_tiles, s, trace_class);
  }
}

// tok_tiles: 4 (up to 64 tokens per block; depth = steps of lookahead, 2 or 4)
// or 8 (128 tokens; 4 steps of lookahead -- at 2 the two resident waves per
// SIMD leave too few registers and it spills)
template <int EPI>
hipError_t launch_wide_epi(const GemmParams &p, int tok_tiles, int depth, hipStream_t s, int trace_class) {
  if (tok_tiles <= 4)
    return depth >= 4 ? launch_wide_d<EPI, 4, 4>(p, s, trace_class) : launch_wide_d<EPI, 4, 2>(p, s, trace_class);
  return launch_wide_d<EPI, 8, 4>(p, s, trace_class);
}

inline hipError_t launch_wide(const GemmParams &p, int tok_tiles, int depth, hipStream_t s, int trace_class) {
  switch (p.epi) {
    case EPI_QKV: return launch_wide_epi<EPI_QKV>(p, tok_tiles, depth, s, trace_class);
    case EPI_RESID: return launch_wide_epi<EPI_RESID>(p, tok_tiles, depth, s, trace_class);
    case EPI_SWIGLU: return launch_wide_epi<EPI_SWIGLU>(p, tok_tiles, depth, s, trace_class);
    default: return launch_wide_epi<EPI_LOGITS>(p, tok_tiles, depth, s, trace_class);
  }
}

// ---------------------------------------------------------------------------
// Square-tiled GEMM for the MFMA-bound range (hundreds of stacked tokens;
// bf16, packed weights).
//
// A workgroup of 8 waves computes 256 weight rows x 256 tokens; wave w owns
// row groups 2 (w % 4), +1 (64 rows) x tokens 128 (w / 4) .. +127, 128
// accumulators.  K advances in half steps of 32: each half step's 16 weight
// fragments and 16 token fragments (1 KiB each, in MFMA lane order) are loaded
// straight into LDS, four per wave, and each wave reads 4 weight and 8 token
// fragments for its 32 MFMAs (384 B of LDS per MFMA; the 256 x 128 tiled
// kernel reads 512).  A ring of four half-step slots, each its own LDS object,
// keeps three half steps in flight; the loop is branch-free (clamped tail
// loads, zero token operand past the end), so the compiler's waits stay
// exact.  The epilogues are the streaming kernel's, and so is the K split
// reduction, which only a tuning override selects (partial tiles through
// memory measured slower than the default choices).
constexpr int kSThreads = 512;
constexpr int kSGroups = 8;     // 32-row groups per workgroup
constexpr int kSTok = 256;      // tokens per workgroup
constexpr int kSStages = 4;
constexpr int kSSlot = 32 * 1024;  // 16 weight + 16 token fragments

template <int EPI>
__global__ __launch_bounds__(kSThreads, 1) void gemm_sq_kernel(GemmParams p) {
  constexpr int D = kSStages - 1;  // half steps in flight
  constexpr int PER = 4;           // loads per wave and half step
  __shared__ __align__(16) unsigned char sl0[kSSlot], sl1[kSSlot], sl2[kSSlot], sl3[kSSlot];
  auto slot_of = [&](auto kc) -> unsigned char * {
    constexpr int k = decltype(kc)::value;
    if constexpr (k == 0) return sl0;
    else if constexpr (k == 1) return sl1;
    else if constexpr (k == 2) return sl2;
    else return sl3;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gq = lane >> 4, l16 = lane & 15;
  const int ntb = (p.T + kSTok - 1) / kSTok;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  // token block fastest (shared weights in L2), then row block, then K split
  const int nrb = (p.nblk + kSGroups - 1) / kSGroups;
  const int tb = wg % ntb, rb = (wg / ntb) % nrb, split = wg / ntb / nrb;
  const int gp = wave & 3, th = wave >> 2;
  // this split's half steps h0 .. h0 + nh - 1
  const int h0 = (int)((long long)split * 2 * p.ksteps / p.splits);
  const int nh = (int)((long long)(split + 1) * 2 * p.ksteps / p.splits) - h0;

  // the four fragments this wave loads each half step: f = wave + 8 i;
  // f < 16: weight fragment (group f / 2, tile f % 2), else token tile f - 16
  const unsigned char *src[PER];
  size_t sstep[PER];  // bytes per full K step (weights: the matrix's step stride; tokens: 128)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = wave + 8 * i;
    if (f < 16) {
      int mi = 0, pr0 = 0;
      if (!map_row(p, rb * kSGroups + (f >> 1), f & 1, 0, mi, pr0)) { mi = 0; pr0 = 0; }
      const size_t g = (size_t)(pr0 / 32);
      const int a = (pr0 / 16) & 1;
      src[i] = static_cast<const unsigned char *>(p.mat[mi].w) + (((g * 2 + a) * 2) * 64 + lane) * 16;
      sstep[i] = (size_t)((p.mat[mi].rows + 31) / 32) * 4096;
    } else {
      const int tt = f - 16;
      src[i] = reinterpret_cast<const unsigned char *>(
          p.x + (size_t)min(tb * kSTok + tt * 16 + l16, p.T - 1) * p.K + 8 * gq);
      sstep[i] = 128;
    }
  }
  // half step h = 2 s + m: weights at s * stride + m * 1 KiB, tokens at s * 128 + m * 64 bytes
  auto issue = [&](int h, auto kc) {
    const int hc = h0 + min(h, nh - 1);
    const int s = hc >> 1, m = hc & 1;
    unsigned char *slot = slot_of(kc);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int f = wave + 8 * i;
      const size_t off = (size_t)s * sstep[i] + (f < 16 ? m * 1024 : m * 64);
      load_lds16(src[i] + off, slot + f * 1024);
    }
  };

  floatx4 acc[2][2][8];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[gi][a][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  static_for<D>([&](auto kc) { issue(decltype(kc)::value, kc); });
  auto step = [&](int h, auto bc) {
    constexpr int later = (D - 1) * PER;
    __builtin_amdgcn_s_waitcnt(0x0F70 | (later & 15) | ((later >> 4) << 14));
    ring_barrier();  // half step h in LDS for everyone; everyone is done with h - 1
    issue(h + D, std::integral_constant<int, (decltype(bc)::value + D) % kSStages>());
    const unsigned char *sl = slot_of(bc);
    bf16x8 wv[2][2];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int a = 0; a < 2; ++a)
        wv[gi][a] = as_bf16x8(ld_v4(sl + (((2 * gp + gi) * 2 + a) * 64 + lane) * 16));
    const bool live = h < nh;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint4 xr = ld_v4(sl + ((16 + th * 8 + j) * 64 + lane) * 16);
      if (!live) xr = uint4{0u, 0u, 0u, 0u};
      const bf16x8 xv = as_bf16x8(xr);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int a = 0; a < 2; ++a) acc[gi][a][j] = mfma16x16x32(wv[gi][a], xv, acc[gi][a][j]);
    }
  };
  for (int hb = 0; hb < nh; hb += kSStages)
    static_for<kSStages>([&](auto kc) { step(hb + decltype(kc)::value, kc); });
  wait_vmem();  // the clamped tail loads

#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int grp = rb * kSGroups + 2 * gp + gi;
    if (grp >= p.nblk || tb * kSTok + th * 128 >= p.T) continue;
    // K splits: the last split to arrive at (group, 128-token block) adds all
    if (p.splits > 1 && !split_reduce<8>(p, acc[gi], grp, tb * 2 + th, split, lane)) continue;
    epilogue<8, EPI>(p, acc[gi], grp, tb * kSTok + th * 128, gq, l16);
  }
}

// The same tiling for packed int4 weights, every load direct-to-LDS (so the
// explicit waits stay exact).  Each ring slot also stages a half step's int4
// codes (16 fragments x 16 rows x 16 bytes: one row's k range of the half
// step) and their group scales.  Each wave issues three loads per half step:
// two token fragments and one 16-byte-per-lane load of: codes of four
// fragments (waves 0-3), the scales of all sixteen (wave 4), a dummy (5-7).  At half step s every
// thread converts half of one (fragment, row) pair of the staged codes of
// s + 1 to bf16 (code - 8 times the scale, as the int4 streaming kernel does)
// after its MFMAs, and writes them in MFMA lane order into that slot's weight
// area (word i of row r goes to lane i * 16 + r); right after the barrier it
// issues the codes of s + 4 and the tokens of s + 3.  The MFMA loop is the bf16 kernel's; the weights cross HBM
// once, as int4.  Weight fragments, token fragments and staging of each slot
// are separate LDS objects: no LDS access then touches an object a
// direct-to-LDS load in flight is writing, and the compiler adds no waits.
constexpr int kS4Stage = 4096 + 512 + 2048;  // codes, scales, dummy

template <int EPI>
__global__ __launch_bounds__(kSThreads, 1) void gemm_sq4_kernel(GemmParams p) {
  constexpr int D = kSStages - 1;  // token half steps in flight
  constexpr int kCodes = 0, kScales = 4096, kJunk = 4096 + 512;
  __shared__ __align__(16) unsigned char w0[16384], w1[16384], w2[16384], w3[16384];
  __shared__ __align__(16) unsigned char t0[16384], t1[16384], t2[16384], t3[16384];
  __shared__ __align__(16) unsigned char g0[kS4Stage], g1[kS4Stage], g2[kS4Stage], g3[kS4Stage];
  auto wslot = [&](auto kc) -> unsigned char * {
    constexpr int k = decltype(kc)::value % kSStages;
    if constexpr (k == 0) return w0;
    else if constexpr (k == 1) return w1;
    else if constexpr (k == 2) return w2;
    else return w3;
  };
  auto tslot = [&](auto kc) -> unsigned char * {
    constexpr int k = decltype(kc)::value % kSStages;
    if constexpr (k == 0) return t0;
    else if constexpr (k == 1) return t1;
    else if constexpr (k == 2) return t2;
    else return t3;
  };
  auto gslot = [&](auto kc) -> unsigned char * {
    constexpr int k = decltype(kc)::value % kSStages;
    if constexpr (k == 0) return g0;
    else if constexpr (k == 1) return g1;
    else if constexpr (k == 2) return g2;
    else return g3;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gq = lane >> 4, l16 = lane & 15;
  const int ntb = (p.T + kSTok - 1) / kSTok;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int nrb = (p.nblk + kSGroups - 1) / kSGroups;
  const int tb = wg % ntb, rb = (wg / ntb) % nrb, split = wg / ntb / nrb;
  const int gp = wave & 3, th = wave >> 2;
  // this split's half steps (of 32; ksteps counts steps of 64) h0 .. h0 + nh - 1
  const int h0 = (int)((long long)split * 2 * p.ksteps / p.splits);
  const int nh = (int)((long long)(split + 1) * 2 * p.ksteps / p.splits) - h0;

  // base of fragment f's int4 data (uint4 units) and scales, and the matrix's
  // step stride (fragments per int4 step of 128)
  auto frag_src = [&](int f, const uint4 *&w, const uint16_t *&sc, size_t &stride) {
    int mi = 0, pr0 = 0;
    if (!map_row(p, rb * kSGroups + (f >> 1), f & 1, 0, mi, pr0)) { mi = 0; pr0 = 0; }
    const size_t base = ((size_t)(pr0 / 32) * 2 + ((pr0 / 16) & 1)) * 64;
    w = static_cast<const uint4 *>(p.mat[mi].w) + base;
    sc = p.mat[mi].s + base;
    stride = (size_t)((p.mat[mi].rows + 31) / 32) * 128;
  };
  // this lane's extra load: bytes at xs + int4 step * xstep + (half step % 4) * xhs
  const unsigned char *xs;
  size_t xstep;
  int xhs, xdst;
  {
    const uint4 *w;
    const uint16_t *sc;
    size_t stride;
    if (wave < 4) {  // codes: fragment 4 wave + lane / 16, row lane % 16
      frag_src(4 * wave + (lane >> 4), w, sc, stride);
      xs = reinterpret_cast<const unsigned char *>(w + l16);
      xstep = stride * 16;
      xhs = 256;
      xdst = kCodes + wave * 1024;
    } else if (wave == 4) {  // scales: fragment (lane % 32) / 2, rows 8 (lane % 2) .. +7
      frag_src((lane & 31) >> 1, w, sc, stride);
      xs = reinterpret_cast<const unsigned char *>(sc + 8 * (lane & 1));
      xstep = stride * 2;
      xhs = 32;
      xdst = kScales + lane * 16;  // lanes 32..63 repeat 0..31 into the dummy area
    } else {  // dummy: any valid bytes
      frag_src(0, w, sc, stride);
      xs = reinterpret_cast<const unsigned char *>(w + l16);
      xstep = 0;
      xhs = 0;
      xdst = kJunk + ((wave - 5) & 1) * 1024;
    }
  }
  auto xissue = [&](int hh, auto kc) {
    const int hc = h0 + min(hh, nh - 1);
    load_lds16(xs + (size_t)(hc >> 2) * xstep + (hc & 3) * xhs, gslot(kc) + xdst);
  };
  // token tiles wave + 8 i
  const unsigned char *tsrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    tsrc[i] = reinterpret_cast<const unsigned char *>(
        p.x + (size_t)min(tb * kSTok + (wave + 8 * i) * 16 + l16, p.T - 1) * p.K + 8 * gq);
  auto tissue = [&](int hh, auto kc) {
    const int hc = h0 + min(hh, nh - 1);
    const int st = hc >> 1, m = hc & 1;
    unsigned char *slot = tslot(kc);
#pragma unroll
    for (int i = 0; i < 2; ++i) load_lds16(tsrc[i] + (size_t)st * 128 + m * 64, slot + (wave + 8 * i) * 1024);
  };
  // conversion: pair (fragment cf, row cr), words 2 ch, 2 ch + 1
  const int pair = threadIdx.x >> 1, ch = threadIdx.x & 1;
  const int cf = pair >> 4, cr = pair & 15;
  auto convert = [&](auto kc) {
    const unsigned char *stg = gslot(kc);
    unsigned char *slot = wslot(kc);
    const uint2 cw = *reinterpret_cast<const uint2 *>(stg + kCodes + (cf * 16 + cr) * 16 + ch * 8);
    const float sc = bf2f(*reinterpret_cast<const uint16_t *>(stg + kScales + (cf * 16 + cr) * 2));
    auto put = [&](uint32_t word, int i) {
      *reinterpret_cast<uint4 *>(slot + cf * 1024 + ((2 * ch + i) * 16 + cr) * 16) =
          __builtin_bit_cast(uint4, dequant8(word, sc));
    };
    put(cw.x, 0);
    put(cw.y, 1);
  };

  floatx4 acc[2][2][8];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[gi][a][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // prologue: half step 0's weights converted; extra(1), tokens(0), extra(2),
  // tokens(1), extra(3), tokens(2) in flight
  xissue(0, std::integral_constant<int, 0>());
  wait_vmem();
  __syncthreads();
  convert(std::integral_constant<int, 0>());
  static_for<D>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    xissue(k + 1, std::integral_constant<int, k + 1>());
    tissue(k, kc);
  });
  // half step s (slot b = s % 4): this wave's tokens of s are in (so are the
  // codes of s + 1, issued before them; 6 loads issued later may remain) and
  // its LDS writes are done; barrier; issue the codes of s + 4 and the tokens
  // of s + 3; compute s; convert s + 1
  auto step = [&](int sh, auto bc) {
    constexpr int b = decltype(bc)::value;
    __builtin_amdgcn_s_waitcnt(0x0070 | 6);
    ring_barrier();
    xissue(sh + 4, std::integral_constant<int, b + 4>());
    tissue(sh + D, std::integral_constant<int, b + D>());
    const unsigned char *wl = wslot(bc), *tl = tslot(bc);
    bf16x8 wv[2][2];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int a = 0; a < 2; ++a)
        wv[gi][a] = as_bf16x8(ld_v4(wl + (((2 * gp + gi) * 2 + a) * 64 + lane) * 16));
    const bool live = sh < nh;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j == 4) __builtin_amdgcn_sched_barrier(0);  // two groups of token reads (register pressure)
      uint4 xr = ld_v4(tl + ((th * 8 + j) * 64 + lane) * 16);
      if (!live) xr = uint4{0u, 0u, 0u, 0u};
      const bf16x8 xv = as_bf16x8(xr);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int a = 0; a < 2; ++a) acc[gi][a][j] = mfma16x16x32(wv[gi][a], xv, acc[gi][a][j]);
    }
    convert(std::integral_constant<int, b + 1>());  // read at s + 1, after its barrier
  };
  for (int hb = 0; hb < nh; hb += kSStages)
    static_for<kSStages>([&](auto kc) { step(hb + decltype(kc)::value, kc); });
  wait_vmem();  // the clamped tail loads

#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int grp = rb * kSGroups + 2 * gp + gi;
    if (grp >= p.nblk || tb * kSTok + th * 128 >= p.T) continue;
    if (p.splits > 1 && !split_reduce<8>(p, acc[gi], grp, tb * 2 + th, split, lane)) continue;
    epilogue<8, EPI>(p, acc[gi], grp, tb * kSTok + th * 128, gq, l16);
  }
}

// Grid of the square-tiled kernels: row blocks x 256-token blocks x K splits.
// With K splits the partial tiles are indexed by 128-token blocks (p.ntblk).
inline int sq_grid(const GemmParams &p) {
  return ((p.nblk + kSGroups - 1) / kSGroups) * ((p.T + kSTok - 1) / kSTok) * p.splits;
}

template <int EPI>
hipError_t launch_sq_epi(const GemmParams &p, hipStream_t s, int trace_class) {
  trace_before(trace_class, s);
  hipLaunchKernelGGL((gemm_sq_kernel<EPI>), dim3(sq_grid(p)), dim3(kSThreads), 0, s, p);
  trace_after(trace_class, s);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_sq4_epi(const GemmParams &p, hipStream_t s, int trace_class) {
  trace_before(trace_class, s);
  hipLaunchKernelGGL((gemm_sq4_kernel<EPI>), dim3(sq_grid(p)), dim3(kSThreads), 0, s, p);
  trace_after(trace_class, s);
  return hipGetLastError();
}

inline hipError_t launch_sq4(const GemmParams &p, hipStream_t s, int trace_class) {
  switch (p.epi) {
    case EPI_QKV: return launch_sq4_epi<EPI_QKV>(p, s, trace_class);
    case EPI_RESID: return launch_sq4_epi<EPI_RESID>(p, s, trace_class);
    case EPI_SWIGLU: return launch_sq4_epi<EPI_SWIGLU>(p, s, trace_class);
    default: return launch_sq4_epi<EPI_LOGITS>(p, s, trace_class);
  }
}

inline hipError_t launch_sq(const GemmParams &p, hipStream_t s, int trace_class) {
  switch (p.epi) {
    case EPI_QKV: return launch_sq_epi<EPI_QKV>(p, s, trace_class);
    case EPI_RESID: return launch_sq_epi<EPI_RESID>(p, s, trace_class);
    case EPI_SWIGLU: return launch_sq_epi<EPI_SWIGLU>(p, s, trace_class);
    default: return launch_sq_epi<EPI_LOGITS>(p, s, trace_class);
  }
}

template <int WT, int TT, int EPI, int G, int KW>
hipError_t launch_g(const GemmParams &p, hipStream_t s, int trace_class) {
  constexpr int WV = waves_per_wg<KW>();
  constexpr int UPW = WV / KW;
  // KW == 1: UPW consecutive row groups per workgroup; else one unit each
  const int nwg = ((p.nblk + UPW - 1) / UPW) * p.splits * p.ntblk;
  trace_before(trace_class, s);
  hipLaunchKernelGGL((gemm_kernel<WT, TT, EPI, G, KW>), dim3(nwg), dim3(64 * WV), 0, s, p);
  trace_after(trace_class, s);
  return hipGetLastError();
}

// (depth, kw) -> instantiation: G = 2 (KW = 1 only), 4 or 8 and KW = 1, 4,
// 8 or 16, within the register budget (gemm_deep_ok, gemm_kw_ok); a request
// outside it takes the nearest smaller setting.
template <int WT, int TT, int EPI, int KW>
hipError_t launch_kw(const GemmParams &p, int depth, hipStream_t s, int trace_class) {
  // KW == 1 also keeps its token ring within kXlMax bytes of LDS
  if constexpr (gemm_deep_ok(WT, TT, KW) && (KW > 1 || xl_bytes<WT, TT, 8>() <= kXlMax)) {
    if (depth >= 8) return launch_g<WT, TT, EPI, 8, KW>(p, s, trace_class);
  }
  if constexpr (KW == 1) {
    if constexpr (xl_bytes<WT, TT, 4>() <= kXlMax) {
      if (depth >= 4) return launch_g<WT, TT, EPI, 4, KW>(p, s, trace_class);
    }
    return launch_g<WT, TT, EPI, 2, KW>(p, s, trace_class);
  } else {
    return launch_g<WT, TT, EPI, 4, KW>(p, s, trace_class);
  }
}

template <int WT, int TT, int EPI>
hipError_t launch_epi(const GemmParams &p, int depth, int kw, hipStream_t s, int trace_class) {
  if constexpr (gemm_kw_ok(WT, TT, 16)) {
    if (kw >= 16) return launch_kw<WT, TT, EPI, 16>(p, depth, s, trace_class);
  }
  if constexpr (gemm_kw_ok(WT, TT, 8)) {
    if (kw >= 8) return launch_kw<WT, TT, EPI, 8>(p, depth, s, trace_class);
  }
  if (kw >= 4) return launch_kw<WT, TT, EPI, 4>(p, depth, s, trace_class);
  return launch_kw<WT, TT, EPI, 1>(p, depth, s, trace_class);
}

template <int WT, int TT>
hipError_t launch_tt(const GemmParams &p, int depth, int kw, hipStream_t s, int trace_class) {
  switch (p.epi) {
    case EPI_QKV: return launch_epi<WT, TT, EPI_QKV>(p, depth, kw, s, trace_class);
    case EPI_RESID: return launch_epi<WT, TT, EPI_RESID>(p, depth, kw, s, trace_class);
    case EPI_SWIGLU: return launch_epi<WT, TT, EPI_SWIGLU>(p, depth, kw, s, trace_class);
    default: return launch_epi<WT, TT, EPI_LOGITS>(p, depth, kw, s, trace_class);
  }
}

template <int WT>
hipError_t launch_wt(const GemmParams &p, int tt, int depth, int kw, hipStream_t s, int tc) {
  switch (tt) {
    case 1: return launch_tt<WT, 1>(p, depth, kw, s, tc);
    case 2: return launch_tt<WT, 2>(p, depth, kw, s, tc);
    case 3: return launch_tt<WT, 3>(p, depth, kw, s, tc);
    default: return launch_tt<WT, 4>(p, depth, kw, s, tc);
  }
}

}  // namespace

}  // namespace sv
