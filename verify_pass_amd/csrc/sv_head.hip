// LM-head softmax finish and token embedding, gfx950.
#include "sv_common.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kEmbedThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

constexpr int kVec = 8;   // float4 loads per thread in flight: 8192 columns per workgroup
constexpr int kStat = 20; // statistics per thread in flight (one round up to 5120 groups)

// (m, s) pairs stand for s * exp(x - m); combining two keeps the larger m.
__device__ __forceinline__ void combine(float &m, float &s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m2 > m) {
    s = s * __builtin_amdgcn_exp2f((m - m2) * kLog2e) + s2;
    m = m2;
  } else {
    s += s2 * __builtin_amdgcn_exp2f((m2 - m) * kLog2e);
  }
}

// M and S of row t: the per-group statistics (group max m_b, group sum of
// exp(l - m_b)) that the LM-head GEMM wrote, token-major so that a row's
// statistics are one contiguous run, combined in a fixed order (every column
// block of the row, and the row statistics kernel, get the same M and S).
// Called by all threads of the workgroup.
__device__ inline void row_stats(const HeadSoftmaxParams &p, int t, float &M, float &S) {
  __shared__ float red_m[kThreads / 64], red_s[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float2 *st = reinterpret_cast<const float2 *>(p.stats) + (size_t)t * p.nblk;
  float m = -INFINITY, s = 0.f;
  // kStat statistics per thread in flight, combined in index order
  for (int b0 = tid; b0 < p.nblk; b0 += kStat * kThreads) {
    float2 e[kStat];
#pragma unroll
    for (int k = 0; k < kStat; ++k) {
      const int b = b0 + k * kThreads;
      e[k] = b < p.nblk ? st[b] : make_float2(-INFINITY, 0.f);
    }
#pragma unroll
    for (int k = 0; k < kStat; ++k) combine(m, s, e[k].x, e[k].y);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    combine(m, s, m2, s2);
  }
  if (lane == 0) {
    red_m[w] = m;
    red_s[w] = s;
  }
  __syncthreads();
  M = red_m[0];
  S = red_s[0];
#pragma unroll
  for (int k = 1; k < kThreads / 64; ++k) combine(M, S, red_m[k], red_s[k]);
}

// Row statistics only (logits stay as they are): one workgroup per row.
__global__ __launch_bounds__(kThreads) void head_rowstats_kernel(HeadSoftmaxParams p) {
  float M, S;
  row_stats(p, blockIdx.x, M, S);
  if (threadIdx.x == 0) {
    p.row_ms[2 * blockIdx.x] = M;
    p.row_ms[2 * blockIdx.x + 1] = S;
  }
}

// p = exp(l - M) / S per row (row_stats), in place.
__global__ __launch_bounds__(kThreads) void head_softmax_kernel(HeadSoftmaxParams p) {
  const int t = blockIdx.y, tid = threadIdx.x;
  float *row = p.logits + (size_t)t * p.V;
  const int c0 = blockIdx.x * p.cols_per_block;
  const int c1 = min(p.V, c0 + p.cols_per_block);
  const bool vec = (p.V & 3) == 0;  // rows are 16-byte aligned: four columns per access
  // this block's logits first: their loads do not depend on the row's M and S
  // and stay in flight while the statistics are combined
  float4 *r4 = reinterpret_cast<float4 *>(row);
  const int e4 = c1 / 4;
  float4 v[kVec];
  if (vec) {
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
      const int c = c0 / 4 + tid + k * kThreads;
      if (c < e4) v[k] = r4[c];
    }
  }
  float M, S;
  row_stats(p, t, M, S);

  const float Mk = M * kLog2e;
  if (vec) {
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
      const int c = c0 / 4 + tid + k * kThreads;
      if (c < e4) {
        float4 o;
        o.x = prob_of_logit(v[k].x, Mk, S);
        o.y = prob_of_logit(v[k].y, Mk, S);
        o.z = prob_of_logit(v[k].z, Mk, S);
        o.w = prob_of_logit(v[k].w, Mk, S);
        r4[c] = o;
      }
    }
  } else {
    for (int c = c0 + tid; c < c1; c += kThreads)
      row[c] = prob_of_logit(row[c], Mk, S);
  }
}

__global__ __launch_bounds__(kEmbedThreads) void embed_kernel(EmbedParams p) {
  const int t = blockIdx.x;
  const int tok = p.tokens[t];
  uint16_t *out = p.out + (size_t)t * p.d;
  if (tok < 0 || tok >= p.V) {
    if (threadIdx.x == 0) set_err(p.err, SV_DEV_ERR_BAD_TOKEN);
    for (int k = threadIdx.x; k < p.d; k += kEmbedThreads) out[k] = 0;
    return;
  }
  if (p.table_bf16) {
    const uint16_t *row = static_cast<const uint16_t *>(p.table) + (size_t)tok * p.d;
    for (int k = threadIdx.x; k < p.d; k += kEmbedThreads) out[k] = row[k];
  } else {
    const float *row = static_cast<const float *>(p.table) + (size_t)tok * p.d;
    for (int k = threadIdx.x; k < p.d; k += kEmbedThreads) out[k] = f2bf(row[k]);
  }
}

}  // namespace

hipError_t launch_head_softmax(const HeadSoftmaxParams &p, hipStream_t s) {
  if (p.cols_per_block != 4 * kThreads * kVec) return hipErrorInvalidValue;
  const dim3 grid((p.V + p.cols_per_block - 1) / p.cols_per_block, p.T);
  trace_before(SV_K_SOFTMAX, s);
  hipLaunchKernelGGL(head_softmax_kernel, grid, dim3(kThreads), 0, s, p);
  trace_after(SV_K_SOFTMAX, s);
  return hipGetLastError();
}

hipError_t launch_head_rowstats(const HeadSoftmaxParams &p, hipStream_t s) {
  trace_before(SV_K_SOFTMAX, s);
  hipLaunchKernelGGL(head_rowstats_kernel, dim3(p.T), dim3(kThreads), 0, s, p);
  trace_after(SV_K_SOFTMAX, s);
  return hipGetLastError();
}

hipError_t launch_embed(const EmbedParams &p, hipStream_t s) {
  trace_before(SV_K_EMBED, s);
  hipLaunchKernelGGL(embed_kernel, dim3(p.T), dim3(kEmbedThreads), 0, s, p);
  trace_after(SV_K_EMBED, s);
  return hipGetLastError();
}

}  // namespace sv
