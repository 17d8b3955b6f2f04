// Ragged causal attention over per-sequence KV caches, gfx950.
//
// Each sequence i brings G * (gamma_i + 1) query rows per KV head (the GQA
// group times its verify tokens) and L_i = kv_len[i] + gamma_i + 1 keys.  Query
// j of sequence i sees keys 0 .. kv_len[i] + j: the causal mask only bites on
// the new keys, and every sequence keeps its own length -- nothing is padded
// to the longest sequence.  Work items are (sequence, key chunk) pairs
// enumerated by a prefix sum over per-sequence chunk counts, times KV heads.
//
// Per wave, 32 keys at a time (values loaded once the keys are used, so the
// two are never live together):
//   S^T[key][row] = K Q^T  (MFMA: keys are M, query rows N, head dim K)
//   online softmax in fp32 (exp2 domain), row max across lanes by shuffles
//   O^T[d][row] += V^T P^T (MFMA: head dim M, query rows N, keys K)
// The key order inside an MFMA is permuted so that the S^T output a lane holds
// (8 consecutive keys of one query row) is exactly the P^T operand it feeds to
// the PV MFMA.  Values are stored in 32-position blocks ([hd][32] per block),
// so that operand is one 16-byte load and a step's values are one contiguous
// 8 KiB run (hd 128).  Waves of a workgroup split the chunk and are combined
// in LDS; each chunk's (o, max, sum) is published with device-scope stores,
// and the last chunk of a (sequence, KV head) to arrive merges all of them by
// log-sum-exp and writes the output rows.
#include <type_traits>
#include <utility>

#include "sv_common.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kKeysPerStep = 32;
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ int dslice(int dg, int gq) {
  // lane group gq covers head-dim columns [64*(dg/2) + 16*gq + 8*(dg%2), +8)
  return 64 * (dg >> 1) + 16 * gq + 8 * (dg & 1);
}

__device__ __forceinline__ void store_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Whether a query row sees key `key` of its sequence (ctx cached keys, then
// the new rows): up to and including its limit lim (-1: a padding row), and
// for token trees (tree set) among the new rows only those its ancestor mask
// names.
__device__ __forceinline__ bool key_visible(int key, int lim, int ctx, bool tree, unsigned long long tm) {
  const int rel = key - ctx;
  return key <= lim && (!tree || rel < 0 || ((tm >> (rel & 63)) & 1ull));
}

// Element (stacked row t, column k of [T][hq * hd]) of the attention output.
__device__ __forceinline__ size_t out_offset(const AttnParams &p, int t, int k) {
  return p.out_ntt > 0 ? frag_index(t, k, p.out_ntt) : (size_t)t * p.hq * p.hd + k;
}

// One step's operands, loaded in two parts so that keys and values are not
// live at the same time: keys (MFMA row m of key tile kt is key
// k0 + 8*(m/4) + 4*kt + m%4), then values (lane (d = 16*dt + l16, gq) holds
// keys k0 + 8*gq .. +7 of head-dim column d).
template <int HD>
__device__ __forceinline__ void load_keys(uint4 (&k)[2][HD / 32], const uint16_t *kbase, int k0, int L, int l16,
                                          int gq) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = min(k0 + 8 * (l16 >> 2) + 4 * kt + (l16 & 3), L - 1);
    const uint16_t *kr = kbase + (size_t)key * HD;
#pragma unroll
    for (int dg = 0; dg < HD / 32; ++dg) k[kt][dg] = *reinterpret_cast<const uint4 *>(kr + dslice(dg, gq));
  }
}

// Eight int8 codes (in memory order) to eight bf16 values (codes are exact in bf16).
__device__ __forceinline__ uint4 codes_to_bf16x8(uint2 c) {
  const uint32_t w[2] = {c.x, c.y};
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t word = w[i >> 1];
    const int sh = (i & 1) * 16;
    const float a = static_cast<float>(static_cast<int8_t>((word >> sh) & 0xFFu));
    const float b = static_cast<float>(static_cast<int8_t>((word >> (sh + 8)) & 0xFFu));
    h[i] = pack_bf16x2(a, b);
  }
  return uint4{h[0], h[1], h[2], h[3]};
}

// int8 caches: the same fragments as load_keys / load_values, one byte per
// value, converted to bf16 codes (the per-position scales are applied to the
// scores and to the probabilities instead).
template <int HD>
__device__ __forceinline__ void load_keys8(uint4 (&k)[2][HD / 32], const int8_t *kbase, int k0, int L, int l16,
                                           int gq) {
  uint2 raw[2][HD / 32];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = min(k0 + 8 * (l16 >> 2) + 4 * kt + (l16 & 3), L - 1);
    const int8_t *kr = kbase + (size_t)key * HD;
#pragma unroll
    for (int dg = 0; dg < HD / 32; ++dg) raw[kt][dg] = *reinterpret_cast<const uint2 *>(kr + dslice(dg, gq));
  }
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int dg = 0; dg < HD / 32; ++dg) k[kt][dg] = codes_to_bf16x8(raw[kt][dg]);
}

template <int HD>
__device__ __forceinline__ void load_values8(uint2 (&v)[HD / 16], const int8_t *vbase, int k0, int l16, int gq) {
  const int8_t *vb = vbase + (size_t)(k0 >> 5) * HD * 32 + 8 * gq;
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt) v[dt] = *reinterpret_cast<const uint2 *>(vb + (dt * 16 + l16) * 32);
}

template <int HD>
__device__ __forceinline__ void load_values(uint4 (&v)[HD / 16], const uint16_t *vbase, int k0, int l16, int gq) {
  // k0 is a multiple of 32 and the block lies inside the cache (cap % 32 == 0)
  const uint16_t *vb = vbase + (size_t)(k0 >> 5) * HD * 32 + 8 * gq;
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt) v[dt] = *reinterpret_cast<const uint4 *>(vb + (dt * 16 + l16) * 32);
}

__device__ __forceinline__ void store_dev2(float *p, float a, float b) {
  __hip_atomic_store(reinterpret_cast<uint64_t *>(p), (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_dev2(const float *p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<float *>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}


// Count this chunk's arrival for (seq, KV head g); the last chunk to arrive
// merges every chunk's (o, max, sum) by log-sum-exp and writes the output
// rows.  Called by all threads once their partial stores are issued.
// qst: the sequence's first stacked row; first, nch: its work items (those
// that were launched: all of them unless the grid was sized for a smaller
// context, which the prep pass flags).
// mw: LDS for 2 * nch * R floats (nch <= 32 chunks, R <= 64 rows); flag: one int.
// The merge is written for memory-level parallelism: the first round of
// partial-row loads (OUTS output pairs x CHUNKS chunks per thread, coherent
// 8-byte loads) is issued together with the loads of every chunk's (max,
// sum); the per-(chunk, row) weights are formed in LDS while they are in
// flight.  The key-split kernel takes 3 x 9 (its 12 query rows x 9 chunks at
// 24 stacked tokens in one round of loads); the query-tiled kernel, whose
// main loop holds more registers, 2 x 12.
template <int HD, int OUTS, int CHUNKS>
__device__ void publish_merge(const AttnParams &p, int qst, int first, int nch, int seq, int g, int R, int n1,
                              int G, int *flag, float *mw) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    int *ctr = p.counters + (size_t)seq * p.hkv + g;
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flag[0] = old == nch - 1;
    if (flag[0]) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!flag[0]) return;

  // partial row (chunk cc, row r) of this (sequence, KV head)
  auto prow = [&](int cc, int r) { return (((size_t)first + cc) * p.hkv + g) * p.rpad + r; };
  constexpr int NP = HD / 2;  // outputs in column pairs: (row r, columns 2 d2, 2 d2 + 1)
  const int nq = R * NP;
  float2 v[OUTS][CHUNKS];
  auto load_round = [&](int q0, int c0) {
#pragma unroll
    for (int u = 0; u < OUTS; ++u) {
      const int q = min(q0 + u * nthr, nq - 1);
      const int r = q / NP, d2 = q - r * NP;
#pragma unroll
      for (int k = 0; k < CHUNKS; ++k) {
        const int cc = min(c0 + k, nch - 1);
        v[u][k] = load_dev2(p.part_o + prow(cc, r) * HD + 2 * d2);
      }
    }
  };
  load_round(tid, 0);  // in flight with the (max, sum) loads below
  float *wm = mw, *wl = mw + nch * R;  // [nch][R] each
  for (int q = tid; q < nch * R; q += nthr) {
    const int cc = q / R, r = q - cc * R;
    const float2 ml = load_dev2(p.part_ml + prow(cc, r) * 2);
    wm[q] = ml.x;
    wl[q] = ml.y;
  }
  __syncthreads();
  // per row: overall max and sum; then each chunk's weight exp2(m_c - M) / sum
  for (int r = tid; r < R; r += nthr) {
    float M = kNegBig;
    for (int cc = 0; cc < nch; ++cc) M = fmaxf(M, wm[cc * R + r]);
    float lt = 0.f;
    for (int cc = 0; cc < nch; ++cc) lt += wl[cc * R + r] * __builtin_amdgcn_exp2f(wm[cc * R + r] - M);
    const float il = lt > 0.f ? 1.f / lt : 0.f;
    for (int cc = 0; cc < nch; ++cc) wm[cc * R + r] = __builtin_amdgcn_exp2f(wm[cc * R + r] - M) * il;
  }
  __syncthreads();
  for (int q0 = tid; q0 < nq; q0 += nthr * OUTS) {
    float2 acc[OUTS];
#pragma unroll
    for (int u = 0; u < OUTS; ++u) acc[u] = make_float2(0.f, 0.f);
    for (int c0 = 0; c0 < nch; c0 += CHUNKS) {
      if (q0 != tid || c0 != 0) load_round(q0, c0);  // the first round is already loaded
#pragma unroll
      for (int u = 0; u < OUTS; ++u) {
        const int r = min(q0 + u * nthr, nq - 1) / NP;
#pragma unroll
        for (int k = 0; k < CHUNKS; ++k) {
          const float w = c0 + k < nch ? wm[(c0 + k) * R + r] : 0.f;
          acc[u].x += v[u][k].x * w;
          acc[u].y += v[u][k].y * w;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < OUTS; ++u) {
      const int q = q0 + u * nthr;
      if (q >= nq) continue;
      const int r = q / NP, d2 = q - r * NP;
      const int hg = r / n1, j = r - hg * n1;
      const int t = qst + j;
      *reinterpret_cast<uint32_t *>(p.out + out_offset(p, t, (g * G + hg) * HD + 2 * d2)) =
          f2bf(acc[u].x) | ((uint32_t)f2bf(acc[u].y) << 16);
    }
  }
}

template <int RT, int HD, bool KV8>
__global__ __launch_bounds__(kThreads, (RT == 1 ? 3 : RT <= 3 ? 2 : 1)) void attn_kernel(AttnParams p) {
  constexpr int NDG = HD / 32;  // MFMA k-groups over the head dim
  constexpr int NDT = HD / 16;  // 16-wide head-dim tiles of the output
  extern __shared__ __align__(16) unsigned char smem[];
  int *flag = reinterpret_cast<int *>(smem);                     // [4]
  float *red_o = reinterpret_cast<float *>(smem + 16);           // [4][HD][16]
  float *red_ml = red_o + 4 * HD * 16;                           // [4][16][2]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, l16 = lane & 15;
  const int g = blockIdx.y;

  const int item = blockIdx.x;
  const int4 ia = p.items[2 * item], ib = p.items[2 * item + 1];
  const int seq = ia.x;
  if (seq < 0) return;
  const int kb = ia.y, ke = ia.z, gam = ia.w, ctx = ib.x, qst = ib.y;
  const int L = ctx + gam + 1;
  if (L > p.kv_cap) {
    // every item of this sequence returns here: no arrivals are counted
    if (tid == 0) set_err(p.err, SV_DEV_ERR_KV_OVERFLOW);
    return;
  }
  const int G = p.hq / p.hkv;
  const int n1 = gam + 1;
  const int R = G * n1;
  const int per_wave = p.chunk / 4;
  const int kw0 = kb + wave * per_wave, kw1 = min(ke, kw0 + per_wave);

  const uint16_t *kbase = static_cast<const uint16_t *>(p.kc[seq]) + (size_t)g * p.kv_cap * HD;
  const uint16_t *vbase = static_cast<const uint16_t *>(p.vc[seq]) + (size_t)g * HD * p.kv_cap;


  // query fragments and per-row causal limits (token trees: ancestor masks)
  const bool tree = p.tree_mask != nullptr;
  bf16x8 qf[RT][NDG];
  int lim[RT];  // last visible key of this lane's row (or -1 for padding rows)
  unsigned long long tm[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rr = rt * 16 + l16;
    tm[rt] = 0ull;
    if (rr < R) {
      const int hg = rr / n1, j = rr - hg * n1;
      const int t = qst + j;
      const uint16_t *q = p.qbuf + ((size_t)t * p.hq + g * G + hg) * HD;
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) qf[rt][dg] = as_bf16x8(*reinterpret_cast<const uint4 *>(q + dslice(dg, gq)));
      lim[rt] = tree ? L - 1 : ctx + j;
      if (tree) tm[rt] = p.tree_mask[t];
    } else {
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) qf[rt][dg] = as_bf16x8(uint4{0u, 0u, 0u, 0u});
      lim[rt] = -1;
    }
  }

  floatx4 o[RT][NDT];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = kNegBig;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[rt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // int8 caches: codes and per-position scales
  const int8_t *kbase8 = KV8 ? static_cast<const int8_t *>(p.kc[seq]) + (size_t)g * p.kv_cap * HD : nullptr;
  const int8_t *vbase8 = KV8 ? static_cast<const int8_t *>(p.vc[seq]) + (size_t)g * HD * p.kv_cap : nullptr;
  const float *ksc = KV8 ? static_cast<const float *>(p.ksc[seq]) + (size_t)g * p.kv_cap : nullptr;
  const float *vsc = KV8 ? static_cast<const float *>(p.vsc[seq]) + (size_t)g * p.kv_cap : nullptr;

  for (int k0 = kw0; k0 < kw1; k0 += kKeysPerStep) {
    uint4 kr[2][NDG];
    uint4 vr[NDT];  // the values in flight with the keys
    float skey[8], sval[8];  // scales of this lane's keys k0 + 8 gq + e (int8 caches)
    if constexpr (KV8) {
      uint2 v8[NDT];
      load_values8<HD>(v8, vbase8, k0, l16, gq);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = min(k0 + 8 * gq + e, L - 1);
        skey[e] = ksc[key];
        sval[e] = vsc[key];
      }
      load_keys8<HD>(kr, kbase8, k0, L, l16, gq);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vr[dt] = codes_to_bf16x8(v8[dt]);
    } else {
      load_keys<HD>(kr, kbase, k0, L, l16, gq);
      load_values<HD>(vr, vbase, k0, l16, gq);
    }
    // scores of every row tile first; the keys are dead afterwards
    floatx4 s[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[rt][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dg = 0; dg < NDG; ++dg) s[rt][kt] = mfma16x16x32(as_bf16x8(kr[kt][dg]), qf[rt][dg], s[rt][kt]);
      }

    bf16x8 pf[RT];
    float alpha[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float sv[8];
      float mx = kNegBig;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = k0 + 8 * gq + e;
        const bool ok = key < kw1 && key_visible(key, lim[rt], ctx, tree, tm[rt]);
        const float raw = KV8 ? s[rt][e >> 2][e & 3] * skey[e] : s[rt][e >> 2][e & 3];
        sv[e] = ok ? raw * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[rt], mx);
      alpha[rt] = __builtin_amdgcn_exp2f(m_run[rt] - m_new);
      float lsum = 0.f;
      uint32_t pb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = __builtin_amdgcn_exp2f(sv[e] - m_new);
        lsum += pe;
        pb[e] = f2bf(KV8 ? pe * sval[e] : pe);  // int8 values: their scale rides on p
      }
      l_run[rt] = l_run[rt] * alpha[rt] + lsum;
      m_run[rt] = m_new;
      pf[rt] = as_bf16x8(uint4{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16), pb[4] | (pb[5] << 16),
                               pb[6] | (pb[7] << 16)});
    }

    // values of keys at or past L are zeroed (the cache holds anything there)
    const int nvalid = L - (k0 + 8 * gq);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint4 v = vr[dt];
      if (nvalid < 8) {
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= nvalid) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        v = uint4{w[0], w[1], w[2], w[3]};
      }
      const bf16x8 vf = as_bf16x8(v);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        o[rt][dt] *= alpha[rt];
        o[rt][dt] = mfma16x16x32(vf, pf[rt], o[rt][dt]);
      }
    }
  }

  // ---- combine the four waves, one row tile at a time; publish the chunk ---
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = l_run[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (gq == 0) {
      red_ml[(wave * 16 + l16) * 2] = m_run[rt];
      red_ml[(wave * 16 + l16) * 2 + 1] = l;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red_o[(wave * HD + dt * 16 + 4 * gq + i) * 16 + l16] = o[rt][dt][i];
    __syncthreads();
    const size_t prow = ((size_t)item * p.hkv + g) * p.rpad + rt * 16;
    for (int idx = tid; idx < HD * 16; idx += kThreads) {
      const int row = idx / HD, d = idx - row * HD;
      if (rt * 16 + row >= R) continue;
      float M = kNegBig;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, red_ml[(w * 16 + row) * 2]);
      float acc = 0.f, lt = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = __builtin_amdgcn_exp2f(red_ml[(w * 16 + row) * 2] - M);
        acc += red_o[(w * HD + d) * 16 + row] * f;
        lt += red_ml[(w * 16 + row) * 2 + 1] * f;
      }
      if (ib.w == 1) {
        // the sequence's keys are this one item: its rows are the output (as
        // the merge of one chunk computes them: o * (1 / l))
        const int rr = rt * 16 + row, hg = rr / n1, j = rr - hg * n1;
        const float il = lt > 0.f ? 1.f / lt : 0.f;
        p.out[out_offset(p, qst + j, (g * G + hg) * HD + d)] = f2bf(acc * il);
        continue;
      }
      store_dev(p.part_o + (prow + row) * HD + d, acc);
      if (d == 0) store_dev2(p.part_ml + (prow + row) * 2, M, lt);
    }
    __syncthreads();
  }

  if (ib.w == 1) return;
  publish_merge<HD, 3, 9>(p, qst, ib.z, ib.w, seq, g, R, n1, G, flag, red_o);  // red_o is free again
}

// ---------------------------------------------------------------------------
// Query-tiled variant for more than 16 query rows per KV head (long drafts,
// wide GQA groups).  Wave w owns query rows 16w .. 16w + 15 over every key of
// the chunk, so no wave holds more than one row tile and no cross-wave
// combine is needed.  Each 32-key step's keys and values are loaded once per
// workgroup straight into LDS in MFMA fragment order (lane l's 16 bytes of
// fragment f at f * 1 KiB + 16 l, read back conflict-free), through a ring of
// three steps so that two are in flight while one is computed.  Each ring slot
// is an LDS object of its own and the step loop is unrolled over the slots
// with no conditional loads: the compiler can then tell that the LDS reads of
// one slot do not alias the direct-to-LDS loads still landing in the others,
// and does not wait for every outstanding load before each step.
constexpr int kQtStages = 3;

// f(std::integral_constant<int, k>()) for k = 0 .. N-1
template <class Fn, int... K>
__device__ __forceinline__ void static_for_impl(Fn &&f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>()), ...);
}
template <int N, class Fn> __device__ __forceinline__ void static_for(Fn &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>());
}

__device__ __forceinline__ void load_lds16(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}
// Workgroup barrier that does not wait for this wave's outstanding loads (the
// waits the ring needs are explicit); the empty asm keeps LDS accesses on
// their side of it.
__device__ __forceinline__ void ring_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// KV8: int8 caches.  Each wave then reads the codes and per-position scales
// of a step straight into registers (the bytes are half those of bf16, and
// the waves of a workgroup read the same lines close together in time, so
// the repeats are served by the vector cache); the scales are applied to the
// scores and to the probabilities as in the key-split kernel.
template <int HD, int NW, bool KV8>
__global__ __launch_bounds__(64 * NW, (NW == 4 ? 2 : 1)) void attn_qt_kernel(AttnParams p) {
  constexpr int NDG = HD / 32, NDT = HD / 16;
  constexpr int F = 2 * NDG + NDT;   // 1 KiB fragments per step: keys (2 x NDG), values (NDT)
  constexpr int FW = F / NW;         // fragments each wave loads per step
  constexpr int SLOT = F * 1024;
  static_assert(F % NW == 0, "fragments must split evenly over the waves");
  static_assert(kQtStages == 3, "three ring slots");
  __shared__ __align__(16) unsigned char ring0[SLOT], ring1[SLOT], ring2[SLOT];
  // the merge's per-(chunk, row) weights: up to 32 chunks x 16 NW rows x 2
  // floats (in the first ring slot when it is large enough)
  constexpr int kMw = kAttnMaxChunks * 16 * NW * 2;
  __shared__ float mw_own[kMw * 4 > SLOT ? kMw : 1];
  __shared__ int flag[4];
  auto slot_of = [&](auto kc) -> unsigned char * {
    constexpr int k = decltype(kc)::value;
    if constexpr (k == 0) return ring0;
    else if constexpr (k == 1) return ring1;
    else return ring2;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, l16 = lane & 15;
  const int g = blockIdx.y;

  const int item = blockIdx.x;
  const int4 ia = p.items[2 * item], ib = p.items[2 * item + 1];
  const int seq = ia.x;
  if (seq < 0) return;
  const int kb = ia.y, ke = ia.z, gam = ia.w, ctx = ib.x, qst = ib.y;
  const int L = ctx + gam + 1;
  if (L > p.kv_cap) {
    if (tid == 0) set_err(p.err, SV_DEV_ERR_KV_OVERFLOW);
    return;
  }
  const int G = p.hq / p.hkv;
  const int n1 = gam + 1;
  const int R = G * n1;
  const int ns = (ke - kb + kKeysPerStep - 1) / kKeysPerStep;
  const bool active = wave * 16 < R;

  const uint16_t *kbase = static_cast<const uint16_t *>(p.kc[seq]) + (size_t)g * p.kv_cap * HD;
  const uint16_t *vbase = static_cast<const uint16_t *>(p.vc[seq]) + (size_t)g * HD * p.kv_cap;
  const int8_t *kbase8 = KV8 ? static_cast<const int8_t *>(p.kc[seq]) + (size_t)g * p.kv_cap * HD : nullptr;
  const int8_t *vbase8 = KV8 ? static_cast<const int8_t *>(p.vc[seq]) + (size_t)g * HD * p.kv_cap : nullptr;
  const float *ksc = KV8 ? static_cast<const float *>(p.ksc[seq]) + (size_t)g * p.kv_cap : nullptr;
  const float *vsc = KV8 ? static_cast<const float *>(p.vsc[seq]) + (size_t)g * p.kv_cap : nullptr;

  // this lane's query fragments and causal limit (row 16 * wave + l16;
  // token trees: its ancestor mask)
  const bool tree = p.tree_mask != nullptr;
  bf16x8 qf[NDG];
  int lim = -1;
  unsigned long long tm = 0ull;
  {
    const int rr = wave * 16 + l16;
    if (rr < R) {
      const int hg = rr / n1, j = rr - hg * n1;
      const uint16_t *q = p.qbuf + ((size_t)(qst + j) * p.hq + g * G + hg) * HD;
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) qf[dg] = as_bf16x8(*reinterpret_cast<const uint4 *>(q + dslice(dg, gq)));
      lim = tree ? L - 1 : ctx + j;
      if (tree) tm = p.tree_mask[qst + j];
    } else {
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) qf[dg] = as_bf16x8(uint4{0u, 0u, 0u, 0u});
    }
  }

  // fragment f = wave + NW i of a step: keys (kt = f / NDG, dg = f % NDG), whose
  // lane rows are keys k0 + 8 (l16 / 4) + 4 kt + l16 % 4 (clamped to the
  // sequence), or values dt = f - 2 NDG (head-dim column 16 dt + l16, keys
  // k0 + 8 gq ..; the 32-key block lies inside the cache)
  // steps past the last reload it (clamped): every step issues the same loads
  auto issue = [&](int st, auto kc) {
    const int k0 = kb + min(st, ns - 1) * kKeysPerStep;
    unsigned char *slot = slot_of(kc);
#pragma unroll
    for (int i = 0; i < FW; ++i) {
      const int f = wave + NW * i;
      const uint16_t *src;
      if (f < 2 * NDG) {
        const int kt = f / NDG, dg = f - kt * NDG;
        const int key = min(k0 + 8 * (l16 >> 2) + 4 * kt + (l16 & 3), L - 1);
        src = kbase + (size_t)key * HD + dslice(dg, gq);
      } else {
        const int dt = f - 2 * NDG;
        src = vbase + (size_t)(k0 >> 5) * HD * 32 + (dt * 16 + l16) * 32 + 8 * gq;
      }
      load_lds16(src, slot + f * 1024);
    }
  };

  floatx4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f;

  // step st (slot b = st % 3): wait for this wave's loads of st (those of
  // st + 1 stay in flight), barrier, issue st + 2 into the slot st - 1 used,
  // compute
  auto step = [&](int st, auto bc) {
    constexpr int b = decltype(bc)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70 | FW);
    ring_barrier();  // every wave's step st is in LDS; every wave is done with step st - 1
    issue(st + 2, std::integral_constant<int, (b + 2) % kQtStages>());
    if (!active || st >= ns) return;
    const unsigned char *sl = slot_of(bc);
    const int k0 = kb + st * kKeysPerStep;
    floatx4 sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sc[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) {
        const uint4 kf = *reinterpret_cast<const uint4 *>(sl + ((kt * NDG + dg) * 64 + lane) * 16);
        sc[kt] = mfma16x16x32(as_bf16x8(kf), qf[dg], sc[kt]);
      }
    }
    float sv[8];
    float mx = kNegBig;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = k0 + 8 * gq + e;
      const bool ok = key < ke && key_visible(key, lim, ctx, tree, tm);
      sv[e] = ok ? sc[e >> 2][e & 3] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float lsum = 0.f;
    uint32_t pb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = __builtin_amdgcn_exp2f(sv[e] - m_new);
      lsum += pe;
      pb[e] = f2bf(pe);
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    const bf16x8 pf = as_bf16x8(uint4{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16), pb[4] | (pb[5] << 16),
                                      pb[6] | (pb[7] << 16)});
    // values of keys at or past L are zeroed (the cache holds anything there)
    const int nvalid = L - (k0 + 8 * gq);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint4 v = *reinterpret_cast<const uint4 *>(sl + ((2 * NDG + dt) * 64 + lane) * 16);
      if (nvalid < 8) {
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= nvalid) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        v = uint4{w[0], w[1], w[2], w[3]};
      }
      o[dt] *= alpha;
      o[dt] = mfma16x16x32(as_bf16x8(v), pf, o[dt]);
    }
  };
  // int8 caches: one step's codes and scales straight from memory
  auto step8 = [&](int st) {
    const int k0 = kb + st * kKeysPerStep;
    uint2 v8[NDT];
    load_values8<HD>(v8, vbase8, k0, l16, gq);
    float skey[8], sval[8];  // scales of this lane's keys k0 + 8 gq + e
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = min(k0 + 8 * gq + e, L - 1);
      skey[e] = ksc[key];
      sval[e] = vsc[key];
    }
    uint4 kr[2][NDG];
    load_keys8<HD>(kr, kbase8, k0, L, l16, gq);
    floatx4 sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sc[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) sc[kt] = mfma16x16x32(as_bf16x8(kr[kt][dg]), qf[dg], sc[kt]);
    }
    float sv[8];
    float mx = kNegBig;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = k0 + 8 * gq + e;
      const bool ok = key < ke && key_visible(key, lim, ctx, tree, tm);
      sv[e] = ok ? sc[e >> 2][e & 3] * skey[e] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[e]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float lsum = 0.f;
    uint32_t pb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = __builtin_amdgcn_exp2f(sv[e] - m_new);
      lsum += pe;
      pb[e] = f2bf(pe * sval[e]);  // the values' scale rides on p
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    const bf16x8 pf = as_bf16x8(uint4{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16), pb[4] | (pb[5] << 16),
                                      pb[6] | (pb[7] << 16)});
    const int nvalid = L - (k0 + 8 * gq);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      uint4 v = codes_to_bf16x8(v8[dt]);
      if (nvalid < 8) {
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= nvalid) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        v = uint4{w[0], w[1], w[2], w[3]};
      }
      o[dt] *= alpha;
      o[dt] = mfma16x16x32(as_bf16x8(v), pf, o[dt]);
    }
  };
  if constexpr (KV8) {
    if (active)
      for (int st = 0; st < ns; ++st) step8(st);
  } else if (ns > 0) {
    issue(0, std::integral_constant<int, 0>());
    issue(1, std::integral_constant<int, 1>());
    for (int st0 = 0; st0 < ns; st0 += kQtStages)
      static_for<kQtStages>([&](auto kc) { step(st0 + decltype(kc)::value, kc); });
    wait_vmem();  // the clamped loads past the last step
  }
  __syncthreads();  // the ring is free for the merge

  if (ib.w == 1) {
    // the sequence's keys are this one item: normalise and write the output
    // rows (as the merge of one chunk computes them: o * (1 / l))
    if (active) {
      float l = l_run;
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      const int row = wave * 16 + l16;
      if (row < R) {
        const float il = l > 0.f ? 1.f / l : 0.f;
        const int hg = row / n1, j = row - hg * n1;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint32_t lo = f2bf(o[dt][0] * il) | ((uint32_t)f2bf(o[dt][1] * il) << 16);
          const uint32_t hi = f2bf(o[dt][2] * il) | ((uint32_t)f2bf(o[dt][3] * il) << 16);
          *reinterpret_cast<uint2 *>(p.out + out_offset(p, qst + j, (g * G + hg) * HD + dt * 16 + 4 * gq)) =
              make_uint2(lo, hi);
        }
      }
    }
    return;
  }

  // publish this chunk's rows: o^T[d][row] (d = 16 dt + 4 gq + i, row = l16)
  if (active) {
    float l = l_run;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int row = wave * 16 + l16;
    if (row < R) {
      const size_t pr = ((size_t)item * p.hkv + g) * p.rpad + row;
      if (gq == 0) store_dev2(p.part_ml + pr * 2, m_run, l);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        store_dev2(p.part_o + pr * HD + dt * 16 + 4 * gq, o[dt][0], o[dt][1]);
        store_dev2(p.part_o + pr * HD + dt * 16 + 4 * gq + 2, o[dt][2], o[dt][3]);
      }
    }
  }
  float *mw = kMw * 4 > SLOT ? mw_own : reinterpret_cast<float *>(ring0);  // the ring is idle now
  publish_merge<HD, 2, 12>(p, qst, ib.z, ib.w, seq, g, R, n1, G, flag, mw);
}

template <int HD, int NW, bool KV8 = false>
hipError_t launch_qt(const AttnParams &p, hipStream_t s) {
  trace_before(SV_K_ATTENTION, s);
  hipLaunchKernelGGL((attn_qt_kernel<HD, NW, KV8>), dim3(p.max_items, p.hkv), dim3(64 * NW), 0, s, p);
  trace_after(SV_K_ATTENTION, s);
  return hipGetLastError();
}

template <int RT, int HD, bool KV8>
hipError_t launch_rt(const AttnParams &p, hipStream_t s) {
  const size_t lds = 16 + (size_t)4 * HD * 16 * sizeof(float) + 4 * 16 * 2 * sizeof(float);
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_kernel<RT, HD, KV8>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  trace_before(SV_K_ATTENTION, s);
  hipLaunchKernelGGL((attn_kernel<RT, HD, KV8>), dim3(p.max_items, p.hkv), dim3(kThreads), lds, s, p);
  trace_after(SV_K_ATTENTION, s);
  return hipGetLastError();
}

// Up to 16 query rows per KV head: waves split the keys (one row tile each);
// more: the query-tiled kernel (one wave per row tile, keys shared in LDS),
// four waves up to 64 rows, eight up to 128.
template <int HD>
hipError_t launch_hd(const AttnParams &p, hipStream_t s) {
  if (p.kv8) {
    if (p.rpad <= 16) return launch_rt<1, HD, true>(p, s);
    return p.rpad <= 64 ? launch_qt<HD, 4, true>(p, s) : launch_qt<HD, 8, true>(p, s);
  }
  if (p.rpad <= 16) return launch_rt<1, HD, false>(p, s);
  if (p.rpad <= 64) return launch_qt<HD, 4>(p, s);
  return launch_qt<HD, 8>(p, s);
}

// The pass's new keys and values into int8 caches: one wave per (token, K or
// V, KV head); scale = absmax / 127 (fp32, correctly rounded), code =
// clamp(rne(x / scale), -127, 127), 0 for an all-zero vector.
template <int HD>
__global__ __launch_bounds__(64) void kv_quant_kernel(KvQuantParams p) {
  const int t = blockIdx.x, which = blockIdx.y / p.hkv, h = blockIdx.y - which * p.hkv;
  const int lane = threadIdx.x;
  const int seq = p.tok_seq[t], pos = p.tok_pos[t];
  if (pos < 0 || pos >= p.kv_cap) return;  // flagged by the QKV pass
  constexpr int PER = HD / 64;
  const uint16_t *src = p.kvstage + (((size_t)t * 2 + which) * p.hkv + h) * HD;
  float x[PER];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    x[i] = bf2f(src[lane + 64 * i]);
    amax = fmaxf(amax, fabsf(x[i]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float scale = __fdiv_rn(amax, 127.f);
  int8_t *codes = static_cast<int8_t *>(which == 0 ? p.kc[seq] : p.vc[seq]);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = lane + 64 * i;
    const float c = amax > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(x[i], scale)), -127.f), 127.f) : 0.f;
    const size_t at = which == 0 ? ((size_t)h * p.kv_cap + pos) * HD + d
                                 : (((size_t)h * (p.kv_cap >> 5) + (pos >> 5)) * HD + d) * 32 + (pos & 31);
    codes[at] = static_cast<int8_t>(c);
  }
  if (lane == 0) static_cast<float *>(which == 0 ? p.ksc[seq] : p.vsc[seq])[(size_t)h * p.kv_cap + pos] = scale;
}

}  // namespace

hipError_t launch_kv_quant(const KvQuantParams &p, hipStream_t s) {
  if (p.hd != 64 && p.hd != 128) return hipErrorInvalidValue;
  if (p.T == 0) return hipSuccess;
  if (p.hd == 64)
    hipLaunchKernelGGL(kv_quant_kernel<64>, dim3(p.T, 2 * p.hkv), dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(kv_quant_kernel<128>, dim3(p.T, 2 * p.hkv), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams &p, hipStream_t s) {
  if (p.kv_cap % 32 || p.chunk % (4 * kKeysPerStep) || p.rpad > kAttnMaxRows) return hipErrorInvalidValue;
  return p.hd == 64 ? launch_hd<64>(p, s) : launch_hd<128>(p, s);
}

}  // namespace sv
