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
#include "sv_common.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kKeysPerStep = 32;
constexpr float kNegBig = -1.0e30f;

// Copy the token map (q_start) and chunk map (chunk_start) of all sequences
// into LDS; returns the total number of work items.
__device__ inline int load_maps(const AttnParams &p, int *qs, int *cs) {
  for (int i = threadIdx.x; i <= p.B; i += blockDim.x) {
    qs[i] = p.q_start[i];
    cs[i] = p.chunk_start[i];
  }
  __syncthreads();
  return cs[p.B];
}

__device__ __forceinline__ int dslice(int dg, int gq) {
  // lane group gq covers head-dim columns [64*(dg/2) + 16*gq + 8*(dg%2), +8)
  return 64 * (dg >> 1) + 16 * gq + 8 * (dg & 1);
}

__device__ __forceinline__ void store_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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

template <int HD>
__device__ __forceinline__ void load_values(uint4 (&v)[HD / 16], const uint16_t *vbase, int k0, int l16, int gq) {
  // k0 is a multiple of 32 and the block lies inside the cache (cap % 32 == 0)
  const uint16_t *vb = vbase + (size_t)(k0 >> 5) * HD * 32 + 8 * gq;
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt) v[dt] = *reinterpret_cast<const uint4 *>(vb + (dt * 16 + l16) * 32);
}

template <int RT, int HD>
__global__ __launch_bounds__(kThreads, (RT == 1 ? 4 : RT <= 3 ? 2 : 1)) void attn_kernel(AttnParams p) {
  constexpr int NDG = HD / 32;  // MFMA k-groups over the head dim
  constexpr int NDT = HD / 16;  // 16-wide head-dim tiles of the output
  extern __shared__ __align__(16) unsigned char smem[];
  int *qs = reinterpret_cast<int *>(smem);
  int *cs = qs + p.B + 1;
  int *flag = cs + p.B + 1;                                      // [2]
  float *red_o = reinterpret_cast<float *>(flag + 2);            // [4][HD][16]
  float *red_ml = red_o + 4 * HD * 16;                           // [4][16][2]
  float *row_m = red_o;                                          // merge: [64] max, [64] 1/sum
  float *row_il = red_o + 64;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gq = lane >> 4, l16 = lane & 15;
  const int g = blockIdx.y;

  const int total = load_maps(p, qs, cs);
  if (blockIdx.x == 0 && g == 0 && tid == 0 && total > p.max_items) set_err(p.err, SV_DEV_ERR_CTX_BOUND);
  const int item = blockIdx.x;
  if (item >= total) return;
  const int seq = upper_index(cs, p.B, item);
  const int c = item - cs[seq];
  const int gam = p.gamma[seq];
  const int ctx = p.kv_len[seq];
  const int L = ctx + gam + 1;
  if (L > p.kv_cap) {
    // every item of this sequence returns here: no arrivals are counted
    if (tid == 0) set_err(p.err, SV_DEV_ERR_KV_OVERFLOW);
    return;
  }
  const int G = p.hq / p.hkv;
  const int n1 = gam + 1;
  const int R = G * n1;
  const int kb = c * p.chunk, ke = min(L, kb + p.chunk);
  const int per_wave = p.chunk / 4;
  const int kw0 = kb + wave * per_wave, kw1 = min(ke, kw0 + per_wave);

  const uint16_t *kbase = static_cast<const uint16_t *>(p.kc[seq]) + (size_t)g * p.kv_cap * HD;
  const uint16_t *vbase = static_cast<const uint16_t *>(p.vc[seq]) + (size_t)g * HD * p.kv_cap;


  // query fragments and per-row causal limits
  bf16x8 qf[RT][NDG];
  int lim[RT];  // last visible key of this lane's row (or -1 for padding rows)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rr = rt * 16 + l16;
    if (rr < R) {
      const int hg = rr / n1, j = rr - hg * n1;
      const int t = qs[seq] + j;
      const uint16_t *q = p.qbuf + ((size_t)t * p.hq + g * G + hg) * HD;
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) qf[rt][dg] = as_bf16x8(*reinterpret_cast<const uint4 *>(q + dslice(dg, gq)));
      lim[rt] = ctx + j;
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

  for (int k0 = kw0; k0 < kw1; k0 += kKeysPerStep) {
    uint4 kr[2][NDG];
    load_keys<HD>(kr, kbase, k0, L, l16, gq);
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
    // values in flight during the softmax arithmetic
    uint4 vr[NDT];
    load_values<HD>(vr, vbase, k0, l16, gq);

    bf16x8 pf[RT];
    float alpha[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float sv[8];
      float mx = kNegBig;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = k0 + 8 * gq + e;
        const bool ok = key < kw1 && key <= lim[rt];
        sv[e] = ok ? s[rt][e >> 2][e & 3] * p.scale_log2 : -INFINITY;
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
        pb[e] = f2bf(pe);
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
      store_dev(p.part_o + (prow + row) * HD + d, acc);
      if (d == 0) {
        store_dev(p.part_ml + (prow + row) * 2, M);
        store_dev(p.part_ml + (prow + row) * 2 + 1, lt);
      }
    }
    __syncthreads();
  }

  // ---- the last chunk of (sequence, KV head) to arrive merges ---------------
  // chunks of this sequence that were launched (all of them unless the grid
  // was sized for a smaller context, which is flagged above)
  const int first = cs[seq];
  const int nch = min(cs[seq + 1], p.max_items) - first;
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

  // per row: overall max and 1 / sum over the chunks
  for (int r = tid; r < R; r += kThreads) {
    float M = kNegBig;
#pragma unroll 8
    for (int cc = 0; cc < nch; ++cc)
      M = fmaxf(M, load_dev(p.part_ml + ((((size_t)first + cc) * p.hkv + g) * p.rpad + r) * 2));
    float lt = 0.f;
#pragma unroll 8
    for (int cc = 0; cc < nch; ++cc) {
      const float *ml = p.part_ml + ((((size_t)first + cc) * p.hkv + g) * p.rpad + r) * 2;
      lt += load_dev(ml + 1) * __builtin_amdgcn_exp2f(load_dev(ml) - M);
    }
    row_m[r] = M;
    row_il[r] = lt > 0.f ? 1.f / lt : 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < R * HD; idx += kThreads) {
    const int r = idx / HD, d = idx - r * HD;
    const float M = row_m[r];
    float acc = 0.f;
#pragma unroll 8
    for (int cc = 0; cc < nch; ++cc) {
      const size_t pr = (((size_t)first + cc) * p.hkv + g) * p.rpad + r;
      acc += load_dev(p.part_o + pr * HD + d) * __builtin_amdgcn_exp2f(load_dev(p.part_ml + pr * 2) - M);
    }
    const int hg = r / n1, j = r - hg * n1;
    const int t = qs[seq] + j;
    p.out[((size_t)t * p.hq + g * G + hg) * HD + d] = f2bf(acc * row_il[r]);
  }
}

template <int RT, int HD>
hipError_t launch_rt(const AttnParams &p, hipStream_t s) {
  const size_t lds = (size_t)(2 * (p.B + 1) + 2) * sizeof(int) + (size_t)4 * HD * 16 * sizeof(float) +
                     4 * 16 * 2 * sizeof(float);
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_kernel<RT, HD>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  trace_before(SV_K_ATTENTION, s);
  hipLaunchKernelGGL((attn_kernel<RT, HD>), dim3(p.max_items, p.hkv), dim3(kThreads), lds, s, p);
  trace_after(SV_K_ATTENTION, s);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_hd(const AttnParams &p, hipStream_t s) {
  switch (p.rpad / 16) {
    case 1: return launch_rt<1, HD>(p, s);
    case 2: return launch_rt<2, HD>(p, s);
    case 3: return launch_rt<3, HD>(p, s);
    default: return launch_rt<4, HD>(p, s);
  }
}

}  // namespace

hipError_t launch_attention(const AttnParams &p, hipStream_t s) {
  if (p.kv_cap % 32 || p.chunk % (4 * kKeysPerStep) || p.rpad > 64) return hipErrorInvalidValue;
  return p.hd == 64 ? launch_hd<64>(p, s) : launch_hd<128>(p, s);
}

}  // namespace sv
