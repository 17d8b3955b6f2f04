// Per-call preparation pass: RMSNorm scales of the input rows and the token map
// (and, when asked, a copy of the input rows in fragment layout).
//
// One workgroup per stacked token t:
//   r[t] = 1 / sqrt(mean(x[t]^2) + eps), summed in a fixed order;
//   (decoder calls) the token's sequence and position: sequence i owns rows
//   q_start[i] .. q_start[i] + gamma_i (q_start = exclusive prefix sum of
//   gamma_i + 1) and row j of it sits at position kv_len[i] + j.
// Workgroup 0 also stores q_start[0..B] and the prefix sum of per-sequence
// attention chunk counts ceil((kv_len[i] + gamma_i + 1) / chunk), and all
// workgroups together write the attention work items (sequence, key range,
// lengths, the sequence's item range), so that an attention workgroup starts
// from one 32-byte load.
// With a rotary table requested, each workgroup also stores cos and sin of
// pos(t) * theta^(-2i/hd) for i < hd/2 (angle and its reduction in fp64).
#include "sv_common.h"

namespace sv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void prep_kernel(PrepParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float red[kThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x;
  // the draft counts and lengths of the first sequences, loaded now so that
  // their latency overlaps the row's
  int g_pre = 0, kv_pre = 0;
  if (p.gamma && tid < p.B) {
    g_pre = p.gamma[tid];
    kv_pre = p.kv_len[tid];
  }
  // sum of squares of row t: each thread a fixed set of 8-element chunks
  const uint16_t *row = p.x + (size_t)t * p.d;
  float s = 0.f;
  for (int c = tid * 8; c < p.d; c += kThreads * 8) {
    const uint4 v = *reinterpret_cast<const uint4 *>(row + c);
    if (p.xp) *reinterpret_cast<uint4 *>(p.xp + frag_index(t, c, p.xp_ntt)) = v;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = __uint_as_float(w[i] << 16), b = __uint_as_float(w[i] & 0xFFFF0000u);
      s += a * a;
      s += b * b;
    }
  }
  // fixed-order reduction: within each wave by shuffles, then the four waves
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    float r = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) r += red[w];
    p.rnorm[t] = 1.f / sqrtf(r / static_cast<float>(p.d) + p.eps);
  }
  if (!p.gamma) return;

  int *qs = reinterpret_cast<int *>(smem);
  int *cs = qs + p.B + 1;
  int *gs = cs + p.B + 1;   // gamma_i
  int *ks = gs + p.B + 1;   // kv_len[i]
  int *tmp = ks + p.B + 1;
  for (int i = tid; i < p.B; i += kThreads) {
    const int g = i < kThreads ? g_pre : p.gamma[i];
    const int kv = i < kThreads ? kv_pre : p.kv_len[i];
    gs[i] = g;
    ks[i] = kv;
    qs[i] = g + 1;
    // a sequence past the host's context bound would need more chunks than
    // the attention merge holds (and than the grid was sized for): it gets no
    // attention work and is flagged; the other sequences are unaffected
    const int nchunks = (kv + g + 1 + p.chunk - 1) / p.chunk;
    const bool over = kv > p.max_ctx || nchunks > kAttnMaxChunks;
    cs[i] = over ? 0 : nchunks;
    if (over && t == 0) set_err(p.err, SV_DEV_ERR_CTX_BOUND);
  }
  __syncthreads();
  const int total_t = block_exscan(qs, p.B, tmp);
  const int total_c = block_exscan(cs, p.B, tmp);
  const int seq = upper_index(qs, p.B, t);
  const int jn = t - qs[seq];               // index of the token in its sequence's chunk
  const int pos = ks[seq] + jn;             // its cache row
  // its position (rotary angle): the row's, or ctx + depth for a tree node,
  // whose ancestor mask the attention reads (the walk up the parent array,
  // staged in LDS: at most 64 nodes)
  int rpos = pos;
  if (p.tree_parent) {
    int *par = tmp + 8;  // block_exscan uses the first four entries
    const int n = gs[seq] + 1;
    for (int j = tid; j < n && j < kMaxTreeNodes; j += kThreads) par[j] = p.tree_parent[qs[seq] + j];
    __syncthreads();
    if (tid == 0) {
      unsigned long long m = 1ull << (jn & 63);
      int depth = 0, v = jn;
      bool bad = jn >= kMaxTreeNodes;
      while (v > 0 && !bad) {
        const int u = par[v];
        if (u < 0 || u >= v) {
          bad = true;
          break;
        }
        m |= 1ull << u;
        v = u;
        ++depth;
      }
      if (bad) {
        set_err(p.err, SV_DEV_ERR_BAD_TREE);
        m = (1ull << (jn & 63)) | 1ull;
      }
      p.tree_mask[t] = m;
      red[0] = __int_as_float(depth);
    }
    __syncthreads();
    rpos = ks[seq] + __float_as_int(red[0]);
  }
  if (tid == 0) {
    p.tok_seq[t] = seq;
    p.tok_pos[t] = pos;
  }
  if (p.rope_cs) {
    // angle pos * theta^(-2i/hd) and its reduction to [-pi, pi] in fp64 (two-part
    // 2 pi), then fp32 sine and cosine of the reduced angle
    constexpr double kTwoPiHi = 6.283185307179586232, kTwoPiLo = 2.449293598294706e-16;
    const int half = p.hd / 2;
    for (int i = tid; i < half; i += kThreads) {
      const double ang = static_cast<double>(rpos) * p.inv_freq[i];
      const double k = rint(ang * (1.0 / kTwoPiHi));
      const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
      float sn, cs;
      sincosf(static_cast<float>(r), &sn, &cs);
      p.rope_cs[((size_t)t * half + i) * 2] = cs;
      p.rope_cs[((size_t)t * half + i) * 2 + 1] = sn;
    }
  }
  if (t == 0) {
    for (int i = tid; i < p.B; i += kThreads) {
      p.q_start[i] = qs[i];
      p.chunk_start[i] = cs[i];
    }
    if (tid == 0) {
      p.q_start[p.B] = total_t;
      p.chunk_start[p.B] = total_c;
      // the attention grid is sized from the host's context bound and the
      // host's draft counts (a device count above them can still overflow it)
      if (total_c > p.max_items) set_err(p.err, SV_DEV_ERR_CTX_BOUND);
    }
  }
  // attention work items, spread over all workgroups: item it is chunk
  // it - cs[seq] of the sequence whose chunk range holds it
  if (p.items) {
    for (int it = t * kThreads + tid; it < p.max_items; it += p.T * kThreads) {
      int4 a = make_int4(-1, 0, 0, 0), b = make_int4(0, 0, 0, 0);
      if (it < total_c) {
        const int sq = upper_index(cs, p.B, it);
        const int g = gs[sq], ctx = ks[sq];
        const int L = ctx + g + 1;
        const int kb = (it - cs[sq]) * p.chunk;
        a = make_int4(sq, kb, min(L, kb + p.chunk), g);
        const int next = sq + 1 < p.B ? cs[sq + 1] : total_c;
        b = make_int4(ctx, qs[sq], cs[sq], min(next, p.max_items) - cs[sq]);
      }
      p.items[2 * it] = a;
      p.items[2 * it + 1] = b;
    }
  }
}

// RMSNorm scales from per-row-group partial sums of squares ([T][nparts], as
// the residual epilogue writes them): one wave per token, the partials added
// in the same order as the GEMM epilogue adds them when it reads them itself
// (lane group gq takes partials gq, gq + 4, ..., then the four groups).
__global__ __launch_bounds__(kThreads) void rnorm_parts_kernel(const float *parts, int nparts, int T, int K,
                                                               float eps, float *rnorm) {
  const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int gq = (threadIdx.x & 63) >> 4;
  const float *pr = parts + (size_t)t * nparts;
  float s = 0.f;
  for (int g = gq; g < nparts; g += 4) s += pr[g];
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  if ((threadIdx.x & 63) == 0) rnorm[t] = 1.f / sqrtf(s / static_cast<float>(K) + eps);
}

}  // namespace

hipError_t launch_rnorm_parts(const float *parts, int nparts, int T, int K, float eps, float *rnorm,
                              hipStream_t s) {
  trace_before(SV_K_PREP, s);
  hipLaunchKernelGGL(rnorm_parts_kernel, dim3((T + 3) / 4), dim3(kThreads), 0, s, parts, nparts, T, K, eps, rnorm);
  trace_after(SV_K_PREP, s);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepParams &p, hipStream_t s) {
  const size_t lds = p.gamma ? (size_t)(4 * (p.B + 1) + 260) * sizeof(int) : 0;
  trace_before(SV_K_PREP, s);
  hipLaunchKernelGGL(prep_kernel, dim3(p.T), dim3(kThreads), lds, s, p);
  trace_after(SV_K_PREP, s);
  return hipGetLastError();
}

}  // namespace sv
