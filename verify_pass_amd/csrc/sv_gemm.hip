// Weight-streaming GEMM over the stacked verify tokens, gfx950.
//
// Y^T[N][T] = W[N][K] * X^T: the weight rows are the MFMA's M side and the
// tokens its N side, so a wave streams 16 weight rows straight from HBM into
// registers (no LDS round trip for the big operand) while the small token
// matrix is staged in LDS and reused by every wave of the workgroup.  One
// read of the weights serves every stacked token, which is the point of a
// verification pass (one weight stream for all drafts of all sequences).
//
// Work decomposition: a workgroup (4 waves) owns a 64-row block of logical
// output rows, one token block of up to 64 tokens and one split of K.  Splits
// write fp32 partial tiles to the workspace; the last split to finish (atomic
// counter per tile) adds them in split order -- so results are bitwise
// repeatable -- and runs the fused epilogue:
//   QKV     RMSNorm scale, RoPE, q to a staging buffer, k/v appended to caches
//   RESID   + residual, bf16 out (O and down projections)
//   SWIGLU  RMSNorm scale, silu(gate) * up, bf16 out
//   LOGITS  RMSNorm scale, fp32 logits, per-block softmax statistics
// RMSNorm needs only a per-token scale r_t = 1/sqrt(mean(x^2) + eps), and
// (r_t x) W = r_t (x W), so the norm is applied in the epilogue from sums of
// squares gathered while the token tiles are staged.
#include "sv_common.h"

namespace sv {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 64;
constexpr int kYStride = 65;        // fp32 epilogue tile row stride (tokens x rows)
constexpr int kStageBytes = 32768;  // LDS bytes for one staged token sub-chunk

// Raw per-lane payload of one K step.
template <int WT> struct Step;
template <> struct Step<WT_BF16> { uint4 v[2]; };
template <> struct Step<WT_F32> { uint4 v[4]; };
template <> struct Step<WT_INT4> { uint4 v; uint32_t s; };

template <int WT> constexpr int kstep() { return WT == WT_INT4 ? 128 : 64; }
template <int WT> constexpr int prefetch() { return WT == WT_F32 ? 2 : 4; }
// K steps per staged token sub-chunk: about kStageBytes of LDS, rounded down
// to whole prefetch groups (at least one group).
template <int WT, int TT> constexpr int stage_steps() {
  constexpr int raw = kStageBytes / (TT * 16 * 2 * kstep<WT>());
  return raw < prefetch<WT>() ? prefetch<WT>() : raw / prefetch<WT>() * prefetch<WT>();
}
template <int WT, int TT> constexpr int x_lds_bytes() {
  return TT * 16 * 2 * kstep<WT>() * stage_steps<WT, TT>();
}

// Lane (row, gq) of step ks covers reduction indices ks*KS + (KS/4)*gq + [0, KS/4).
template <int WT>
__device__ __forceinline__ Step<WT> load_step(const void *w, const uint16_t *sc, int row, int K,
                                              int ks, int gq) {
  Step<WT> r;
  if constexpr (WT == WT_BF16) {
    const uint16_t *b = static_cast<const uint16_t *>(w) + (size_t)row * K + ks * 64 + 16 * gq;
    r.v[0] = *reinterpret_cast<const uint4 *>(b);
    r.v[1] = *reinterpret_cast<const uint4 *>(b + 8);
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

// int4 word (8 codes, offset by 8) times the group scale, to bf16.
__device__ __forceinline__ bf16x8 dequant8(uint32_t word, float s) {
  uint4 o;
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = static_cast<float>(static_cast<int>((word >> (4 * e)) & 15u) - 8) * s;
    h[e] = f2bf(v);
  }
  o.x = h[0] | (h[1] << 16);
  o.y = h[2] | (h[3] << 16);
  o.z = h[4] | (h[5] << 16);
  o.w = h[6] | (h[7] << 16);
  return as_bf16x8(o);
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
  uint4 ho{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  uint4 lw{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
  hi = as_bf16x8(ho);
  lo = as_bf16x8(lw);
}

// Logical row lr of block blk -> (matrix, physical row).  False past the end.
__device__ __forceinline__ bool map_row(const GemmParams &p, int blk, int lr, int &m, int &pr) {
  if (p.rowmap == RM_SWIGLU) {
    const int f = blk * 32 + (lr & 31);
    if (f >= p.mat[0].rows) return false;
    m = lr < 32 ? 0 : 1;
    pr = f;
    return true;
  }
  int n;
  if (p.rowmap == RM_ROPE_PAIRS) {
    const int bph = p.hd / 64;
    const int head = blk / bph, hb = blk - head * bph;
    n = head * p.hd + (lr < 32 ? 32 * hb + lr : p.hd / 2 + 32 * hb + lr - 32);
  } else {
    n = blk * kRowsPerBlock + lr;
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

// Swizzled LDS offset (elements) of the 16-byte chunk holding column c of row r.
__device__ __forceinline__ int xs_off(int r, int c, int cols) {
  const int chunk = (c >> 3) ^ (r & 7);
  return r * cols + (chunk << 3) + (c & 7);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Bijective remap of the dispatch index so that consecutive logical tiles run
// on the same XCD (dispatch is round-robin over the 8 XCDs).
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  const int q = nwg / 8, r = nwg % 8;
  const int x = wg % 8, k = wg / 8;
  return x * q + min(x, r) + k;
}

template <int WT, int TT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int KS = kstep<WT>();
  constexpr int NTOK = TT * 16;
  constexpr int SS = stage_steps<WT, TT>();           // steps per staged sub-chunk
  constexpr int SCOLS = SS * KS;                      // staged columns
  constexpr int P = prefetch<WT>();                   // weight prefetch depth (steps)
  static_assert(SS >= 1 && SS % P == 0, "stage must hold whole prefetch groups");

  __shared__ float ss4[256];
  __shared__ float ssv[64];
  __shared__ int flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, l16 = lane & 15;
  const int nwg = gridDim.x;
  int lid = xcd_remap(blockIdx.x, nwg);
  const int tb = lid % p.ntblk;
  lid /= p.ntblk;
  const int split = lid % p.splits;
  const int blk = lid / p.splits;
  const int t0 = tb * NTOK;
  const int s0 = (int)((long long)split * p.ksteps / p.splits);
  const int s1 = (int)((long long)(split + 1) * p.ksteps / p.splits);
  const int nsteps = s1 - s0;

  // This lane's weight row (loads); out-of-range rows read row 0 and are dropped.
  int mi = 0, pr = 0;
  if (!map_row(p, blk, wave * 16 + l16, mi, pr)) { mi = 0; pr = 0; }
  const void *wbase = p.mat[mi].w;
  const uint16_t *sbase = p.mat[mi].s;

  floatx4 acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};

  Step<WT> buf[P];
  if (nsteps > 0) {
#pragma unroll
    for (int j = 0; j < P; ++j) buf[j] = load_step<WT>(wbase, sbase, pr, p.K, s0 + min(j, nsteps - 1), gq);
  }

  uint16_t *xs = reinterpret_cast<uint16_t *>(smem);
  float ssum = 0.f;  // this thread's share of one token row's sum of squares
  const int ss_row = tid >> 2, ss_part = tid & 3;

  for (int st0 = 0; st0 < nsteps; st0 += SS) {
    const int nst = min(SS, nsteps - st0);
    const int cols = nst * KS;
    __syncthreads();
    // stage X[t0 .. t0+NTOK)[ (s0+st0)*KS .. + cols ) into LDS (zero past T)
    const int cpr = cols / 8;
    for (int idx = tid; idx < NTOK * cpr; idx += kThreads) {
      const int r = idx / cpr, c8 = idx - r * cpr;
      uint4 v{0u, 0u, 0u, 0u};
      if (t0 + r < p.T)
        v = *reinterpret_cast<const uint4 *>(p.x + (size_t)(t0 + r) * p.K + (s0 + st0) * KS + c8 * 8);
      *reinterpret_cast<uint4 *>(xs + xs_off(r, c8 * 8, SCOLS)) = v;
    }
    __syncthreads();
    if (p.norm && ss_row < NTOK) {
      const int q4 = cols / 4;
      float s = 0.f;
      for (int c = ss_part * q4; c < (ss_part + 1) * q4; ++c) {
        const float f = bf2f(xs[xs_off(ss_row, c, SCOLS)]);
        s += f * f;
      }
      ssum += s;
    }
    // K loop over the staged columns with a rolling prefetch of P weight steps.
    for (int b = 0; b < nst; b += P) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int st = st0 + b + j;
        if (b + j < nst) {
          const int cbase = (b + j) * KS + (KS / 4) * gq;
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            const int r = tt * 16 + l16;
            if constexpr (WT == WT_BF16) {
#pragma unroll
              for (int m = 0; m < 2; ++m) {
                const bf16x8 bx = as_bf16x8(*reinterpret_cast<const uint4 *>(xs + xs_off(r, cbase + 8 * m, SCOLS)));
                acc[tt] = mfma16x16x32(as_bf16x8(buf[j].v[m]), bx, acc[tt]);
              }
            } else if constexpr (WT == WT_INT4) {
              const float s = bf2f(static_cast<uint16_t>(buf[j].s));
              const uint32_t wv[4] = {buf[j].v.x, buf[j].v.y, buf[j].v.z, buf[j].v.w};
#pragma unroll
              for (int m = 0; m < 4; ++m) {
                const bf16x8 bx = as_bf16x8(*reinterpret_cast<const uint4 *>(xs + xs_off(r, cbase + 8 * m, SCOLS)));
                acc[tt] = mfma16x16x32(dequant8(wv[m], s), bx, acc[tt]);
              }
            } else {
#pragma unroll
              for (int m = 0; m < 2; ++m) {
                const bf16x8 bx = as_bf16x8(*reinterpret_cast<const uint4 *>(xs + xs_off(r, cbase + 8 * m, SCOLS)));
                bf16x8 hi, lo;
                split8(buf[j].v[2 * m], buf[j].v[2 * m + 1], hi, lo);
                acc[tt] = mfma16x16x32(hi, bx, acc[tt]);
                acc[tt] = mfma16x16x32(lo, bx, acc[tt]);
              }
            }
          }
        }
        buf[j] = load_step<WT>(wbase, sbase, pr, p.K, s0 + min(st + P, nsteps - 1), gq);
      }
    }
  }
  __syncthreads();

  // ---- gather this split's tile into LDS: Y[t][lr] -------------------------
  float *ys = reinterpret_cast<float *>(smem);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) ys[(tt * 16 + l16) * kYStride + wave * 16 + 4 * gq + i] = acc[tt][i];
  if (p.norm) {
    ss4[tid] = ssum;
    __syncthreads();
    if (tid < NTOK) ssv[tid] = ((ss4[4 * tid] + ss4[4 * tid + 1]) + ss4[4 * tid + 2]) + ss4[4 * tid + 3];
  }
  __syncthreads();

  if (p.splits > 1) {
    const size_t tile = (size_t)NTOK * kRowsPerBlock;
    float *mine = p.partial + (((size_t)split * p.nblk + blk) * p.ntblk + tb) * tile;
    for (int idx = tid; idx < NTOK * kRowsPerBlock; idx += kThreads)
      mine[idx] = ys[(idx >> 6) * kYStride + (idx & 63)];
    if (p.norm && tid < NTOK)
      p.part_ss[(((size_t)blk * p.splits + split) * p.ntblk + tb) * 64 + tid] = ssv[tid];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      int *ctr = p.counters + (size_t)blk * p.ntblk + tb;
      const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      flag = (old == p.splits - 1);
      if (flag) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!flag) return;
    __threadfence();
    for (int idx = tid; idx < NTOK * kRowsPerBlock; idx += kThreads) {
      float s = 0.f;
      for (int sp = 0; sp < p.splits; ++sp)
        s += __builtin_nontemporal_load(p.partial + (((size_t)sp * p.nblk + blk) * p.ntblk + tb) * tile + idx);
      ys[(idx >> 6) * kYStride + (idx & 63)] = s;
    }
    if (p.norm && tid < NTOK) {
      float s = 0.f;
      for (int sp = 0; sp < p.splits; ++sp)
        s += __builtin_nontemporal_load(p.part_ss + (((size_t)blk * p.splits + sp) * p.ntblk + tb) * 64 + tid);
      ssv[tid] = s;
    }
    __syncthreads();
  }

  // per-token RMSNorm scale
  if (tid < NTOK) {
    float r = 1.f;
    if (p.norm) r = 1.f / sqrtf(ssv[tid] / static_cast<float>(p.K) + p.eps);
    ss4[tid] = r;
  }
  __syncthreads();
  const float *rt = ss4;

  // ---- fused epilogues ------------------------------------------------------
  if (p.epi == EPI_RESID) {
    uint16_t *out = static_cast<uint16_t *>(p.out);
    for (int idx = tid; idx < NTOK * kRowsPerBlock; idx += kThreads) {
      const int t = idx >> 6, lr = idx & 63, n = blk * kRowsPerBlock + lr;
      if (t0 + t < p.T && n < p.N) {
        const size_t o = (size_t)(t0 + t) * p.ldo + n;
        out[o] = f2bf(ys[t * kYStride + lr] * rt[t] + bf2f(p.resid[o]));
      }
    }
  } else if (p.epi == EPI_SWIGLU) {
    uint16_t *out = static_cast<uint16_t *>(p.out);
    for (int idx = tid; idx < NTOK * 32; idx += kThreads) {
      const int t = idx >> 5, lr = idx & 31, f = blk * 32 + lr;
      if (t0 + t < p.T && f < p.mat[0].rows) {
        const float g = ys[t * kYStride + lr] * rt[t];
        const float u = ys[t * kYStride + lr + 32] * rt[t];
        const float sig = 1.f / (1.f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
        out[(size_t)(t0 + t) * p.ldo + f] = f2bf(g * sig * u);
      }
    }
  } else if (p.epi == EPI_LOGITS) {
    float *out = static_cast<float *>(p.out);
    const int n = blk * kRowsPerBlock + lane;
    const bool valid = n < p.N;
    for (int t = wave; t < NTOK; t += 4) {
      if (t0 + t >= p.T) break;
      const float v = ys[t * kYStride + lane] * rt[t];
      if (valid) out[(size_t)(t0 + t) * p.ldo + n] = v;
      const float m = wave_max(valid ? v : -INFINITY);
      const float e = valid ? __builtin_amdgcn_exp2f((v - m) * 1.4426950408889634f) : 0.f;
      const float s = wave_sum(e);
      if (lane == 0) {
        float *st = p.stats + ((size_t)blk * p.T + t0 + t) * 2;
        st[0] = m;
        st[1] = s;
      }
    }
  } else {  // EPI_QKV
    int *gam = reinterpret_cast<int *>(smem + NTOK * kYStride * sizeof(float));
    int *tmp = gam + (p.B + 1);
    for (int i = tid; i < p.B; i += kThreads) gam[i] = p.gamma[i] + 1;
    __syncthreads();
    block_exscan(gam, p.B, tmp);
    const int bph = p.hd / 64;
    const int head = blk / bph, hb = blk - head * bph;
    const int half = p.hd / 2;
    for (int idx = tid; idx < NTOK * 32; idx += kThreads) {
      const int t = idx >> 5, lr = idx & 31;
      const int tg = t0 + t;
      if (tg >= p.T) continue;
      const int seq = upper_index(gam, p.B, tg);
      const int pos = p.kv_len[seq] + (tg - gam[seq]);
      const int i = 32 * hb + lr;  // rotation pair (i, i + hd/2)
      const float a = ys[t * kYStride + lr] * rt[t];
      const float b = ys[t * kYStride + lr + 32] * rt[t];
      if (head < p.hq + p.hkv) {
        const double inv = pow(static_cast<double>(p.rope_theta), -2.0 * i / p.hd);
        double sn, cs;
        sincos(static_cast<double>(pos) * inv, &sn, &cs);
        const float c = static_cast<float>(cs), s = static_cast<float>(sn);
        const float ra = a * c - b * s, rb = b * c + a * s;
        if (head < p.hq) {
          uint16_t *q = p.qbuf + ((size_t)tg * p.hq + head) * p.hd;
          q[i] = f2bf(ra);
          q[i + half] = f2bf(rb);
        } else {
          if (pos >= p.kv_cap || pos < 0) { set_err(p.err, SV_DEV_ERR_KV_OVERFLOW); continue; }
          uint16_t *k = static_cast<uint16_t *>(p.kc[seq]) + ((size_t)(head - p.hq) * p.kv_cap + pos) * p.hd;
          k[i] = f2bf(ra);
          k[i + half] = f2bf(rb);
        }
      } else {
        if (pos >= p.kv_cap || pos < 0) { set_err(p.err, SV_DEV_ERR_KV_OVERFLOW); continue; }
        uint16_t *v = static_cast<uint16_t *>(p.vc[seq]) + (size_t)(head - p.hq - p.hkv) * p.hd * p.kv_cap;
        v[(size_t)i * p.kv_cap + pos] = f2bf(a);
        v[(size_t)(i + half) * p.kv_cap + pos] = f2bf(b);
      }
    }
  }
}

template <int WT, int TT>
hipError_t launch_tt(const GemmParams &p, hipStream_t s, int trace_class) {
  const int nwg = p.nblk * p.splits * p.ntblk;
  size_t lds = x_lds_bytes<WT, TT>();
  const size_t ylds = (size_t)TT * 16 * kYStride * sizeof(float);
  size_t need = ylds + (p.epi == EPI_QKV ? (size_t)(p.B + 1 + 257) * sizeof(int) : 0);
  if (need > lds) lds = need;
  if (lds > 65536) {
    hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_kernel<WT, TT>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  }
  trace_before(trace_class, s);
  hipLaunchKernelGGL((gemm_kernel<WT, TT>), dim3(nwg), dim3(kThreads), lds, s, p);
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

}  // namespace sv
