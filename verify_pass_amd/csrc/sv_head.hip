// LM-head softmax finish and token embedding, gfx950.
#include "sv_common.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// p = exp(l - M) / S per row, where M and S combine the per-group statistics
// (group max m_b, group sum of exp(l - m_b)) that the LM-head GEMM wrote,
// token-major so that a row's statistics are one contiguous run.  They are
// reduced in a fixed order, so every column block of a row computes the same
// M and S.
__device__ inline float block_max(float v, float *red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__device__ inline float block_sum(float v, float *red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void head_softmax_kernel(HeadSoftmaxParams p) {
  __shared__ float red[kThreads];
  const int t = blockIdx.y, tid = threadIdx.x;
  const float2 *st = reinterpret_cast<const float2 *>(p.stats) + (size_t)t * p.nblk;
  float m = -INFINITY;
  for (int b = tid; b < p.nblk; b += kThreads) m = fmaxf(m, st[b].x);
  const float M = block_max(m, red);
  float s = 0.f;
  for (int b = tid; b < p.nblk; b += kThreads) {
    const float2 e = st[b];
    s += e.y * __builtin_amdgcn_exp2f((e.x - M) * kLog2e);
  }
  const float S = block_sum(s, red);
  float *row = p.logits + (size_t)t * p.V;
  const int c0 = blockIdx.x * p.cols_per_block;
  const int c1 = min(p.V, c0 + p.cols_per_block);
  const float Mk = M * kLog2e;
  if ((p.V & 3) == 0) {  // rows are 16-byte aligned: four columns per load
    float4 *r4 = reinterpret_cast<float4 *>(row);
    for (int c = c0 / 4 + tid; c < c1 / 4; c += kThreads) {
      float4 v = r4[c];
      v.x = __builtin_amdgcn_exp2f(fmaf(v.x, kLog2e, -Mk)) / S;
      v.y = __builtin_amdgcn_exp2f(fmaf(v.y, kLog2e, -Mk)) / S;
      v.z = __builtin_amdgcn_exp2f(fmaf(v.z, kLog2e, -Mk)) / S;
      v.w = __builtin_amdgcn_exp2f(fmaf(v.w, kLog2e, -Mk)) / S;
      r4[c] = v;
    }
  } else {
    for (int c = c0 + tid; c < c1; c += kThreads)
      row[c] = __builtin_amdgcn_exp2f(fmaf(row[c], kLog2e, -Mk)) / S;
  }
}

__global__ __launch_bounds__(kThreads) void embed_kernel(EmbedParams p) {
  const int t = blockIdx.x;
  const int tok = p.tokens[t];
  uint16_t *out = p.out + (size_t)t * p.d;
  if (tok < 0 || tok >= p.V) {
    if (threadIdx.x == 0) set_err(p.err, SV_DEV_ERR_BAD_TOKEN);
    for (int k = threadIdx.x; k < p.d; k += kThreads) out[k] = 0;
    return;
  }
  if (p.table_bf16) {
    const uint16_t *row = static_cast<const uint16_t *>(p.table) + (size_t)tok * p.d;
    for (int k = threadIdx.x; k < p.d; k += kThreads) out[k] = row[k];
  } else {
    const float *row = static_cast<const float *>(p.table) + (size_t)tok * p.d;
    for (int k = threadIdx.x; k < p.d; k += kThreads) out[k] = f2bf(row[k]);
  }
}

}  // namespace

hipError_t launch_head_softmax(const HeadSoftmaxParams &p, hipStream_t s) {
  const dim3 grid((p.V + p.cols_per_block - 1) / p.cols_per_block, p.T);
  trace_before(SV_K_SOFTMAX, s);
  hipLaunchKernelGGL(head_softmax_kernel, grid, dim3(kThreads), 0, s, p);
  trace_after(SV_K_SOFTMAX, s);
  return hipGetLastError();
}

hipError_t launch_embed(const EmbedParams &p, hipStream_t s) {
  trace_before(SV_K_EMBED, s);
  hipLaunchKernelGGL(embed_kernel, dim3(p.T), dim3(kThreads), 0, s, p);
  trace_after(SV_K_EMBED, s);
  return hipGetLastError();
}

}  // namespace sv
