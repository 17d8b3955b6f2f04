// Acceptance, resampling and KV-length commit, gfx950.
//
// Rejection sampling in the sense of Leviathan, Kalman and Matias keeps the
// output distribution of plain decoding; the verifier keeps the drafts up to
// the first rejection and adds one token of its own.  Draws use integer
// weights R(x) = trunc(fl32(r(x) * 2^32)): sums of integers do not depend on
// the order in which lanes and workgroups add them, so the token drawn for a
// given uniform is the same on any grid shape.
//
// One kernel, grid = vocabulary chunks x sequences.  Every workgroup of a
// sequence reduces its chunk (stochastic: the acceptance tests, then integer
// weight sums of the resampling row and of the fallback target row and the
// chunk argmax; greedy: the chunk argmax of each of the sequence's target
// rows), publishes the result with device-scope stores and counts its
// arrival.  The last workgroup to arrive combines the chunk results with
// block-wide reductions and scans, and commits.
#include "sv_common.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesA = kThreads / 64;
constexpr int kSegMax = 32;  // chunk / kThreads: elements per thread in the exact scan
constexpr int kVecA = kSegMax / 4;  // float4 loads per thread and row over a chunk
constexpr float kTwo32 = 4294967296.0f;

typedef unsigned long long u64;

__device__ __forceinline__ u64 weight_of(float r) {
  r = fmaxf(r, 0.f);
  return static_cast<u64>(r * kTwo32);
}

// argmax combine: larger value wins, lower index on ties (order-independent)
__device__ __forceinline__ void amax(float &v, int &i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// Probabilities of one row as the rule reads them: the entries themselves, or
// (logits mode) formed from the row's logits and (max, sum) exactly as the
// head's softmax finish forms them.
struct PXf {
  bool on;
  float Mk, S;
  __device__ __forceinline__ float operator()(float v) const { return on ? prob_of_logit(v, Mk, S) : v; }
  __device__ __forceinline__ float4 operator()(float4 v) const {
    return on ? make_float4(prob_of_logit(v.x, Mk, S), prob_of_logit(v.y, Mk, S), prob_of_logit(v.z, Mk, S),
                            prob_of_logit(v.w, Mk, S))
              : v;
  }
};
__device__ __forceinline__ PXf pxf_of(const AcceptParams &p, int row) {
  if (!p.row_ms) return PXf{false, 0.f, 1.f};
  return PXf{true, p.row_ms[2 * row] * kLog2eF, p.row_ms[2 * row + 1]};
}

struct Shared {
  u64 a[kWavesA], b[kWavesA];
  float v[kWavesA];
  int i[kWavesA];
  int first_fail, bad, flag, found, chunk_hit, result;
  u64 target;
};

// Block-wide sums of two u64 values and an argmax; every thread gets the result.
__device__ inline void block_reduce(u64 &a, u64 &b, float &v, int &ix, Shared &sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
    const float v2 = __shfl_xor(v, o);
    const int i2 = __shfl_xor(ix, o);
    amax(v, ix, v2, i2);
  }
  if (lane == 0) {
    sh.a[w] = a;
    sh.b[w] = b;
    sh.v[w] = v;
    sh.i[w] = ix;
  }
  __syncthreads();
  a = 0;
  b = 0;
  v = -INFINITY;
  ix = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < kWavesA; ++k) {
    a += sh.a[k];
    b += sh.b[k];
    amax(v, ix, sh.v[k], sh.i[k]);
  }
  __syncthreads();
}

// Exclusive prefix sum over the block in thread order; *total gets the sum.
__device__ inline u64 block_exscan(u64 v, u64 *total, Shared &sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  u64 inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh.a[w] = inc;
  __syncthreads();
  u64 before = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kWavesA; ++k) {
    if (k < w) before += sh.a[k];
    tot += sh.a[k];
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

// Device-scope (cross-XCD coherent) stores and loads of the chunk results.
__device__ __forceinline__ void put_part(AcceptPart *p, u64 sres, u64 sp, float mv, int mi) {
  u64 *w = reinterpret_cast<u64 *>(p);
  __hip_atomic_store(w, sres, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(w + 1, sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const u64 mx = (static_cast<u64>(static_cast<uint32_t>(mi)) << 32) | __float_as_uint(mv);
  __hip_atomic_store(w + 2, mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ AcceptPart get_part(const AcceptPart *p) {
  u64 *w = reinterpret_cast<u64 *>(const_cast<AcceptPart *>(p));
  AcceptPart v;
  v.sum_res = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.sum_p = __hip_atomic_load(w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const u64 mx = __hip_atomic_load(w + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.max_p = __uint_as_float(static_cast<uint32_t>(mx));
  v.arg_p = static_cast<int>(mx >> 32);
  return v;
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Count this workgroup's arrival after its results are stored; true for the
// last of `expected` (which resets the counter for the next call).
__device__ inline bool arrive_last(int *ctr, int expected, Shared &sh) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.flag = old == expected - 1;
    if (sh.flag) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return sh.flag != 0;
}

// q_start of sequence i: sum of gamma_k + 1 over k < i.
__device__ inline int seq_start(const int *gamma, int i, Shared &sh) {
  u64 s = 0, z = 0;
  for (int k = threadIdx.x; k < i; k += kThreads) s += gamma[k] + 1;
  float v = 0.f;
  int ix = 0;
  block_reduce(s, z, v, ix, sh);
  return static_cast<int>(s);
}

// This thread's share of the argmax of row[x0, x1).
__device__ inline void chunk_argmax(const float *row, PXf xf, int x0, int x1, bool vec, float &bv, int &bi) {
  bv = -INFINITY;
  bi = 0x7fffffff;
  if (vec) {
    const float4 *r4 = reinterpret_cast<const float4 *>(row);
    float4 v[kVecA];
#pragma unroll
    for (int k = 0; k < kVecA; ++k) {
      const int x = x0 / 4 + threadIdx.x + k * kThreads;
      v[k] = x < x1 / 4 ? xf(r4[x]) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int k = 0; k < kVecA; ++k) {
      const int x = x0 / 4 + threadIdx.x + k * kThreads;
      if (x >= x1 / 4) continue;
      amax(bv, bi, v[k].x, 4 * x);
      amax(bv, bi, v[k].y, 4 * x + 1);
      amax(bv, bi, v[k].z, 4 * x + 2);
      amax(bv, bi, v[k].w, 4 * x + 3);
    }
  } else {
    for (int x = x0 + threadIdx.x; x < x1; x += kThreads) amax(bv, bi, xf(row[x]), x);
  }
}

__device__ inline void commit_bad(const AcceptParams &p, int i) {
  p.accepted[i] = -1;
  p.next_token[i] = -1;
  set_err(p.err, SV_DEV_ERR_BAD_TOKEN);
}

__global__ __launch_bounds__(kThreads) void accept_kernel(AcceptParams p) {
  __shared__ Shared sh;
  const int tid = threadIdx.x, c = blockIdx.x, i = blockIdx.y;
  const int x0 = c * p.chunk, x1 = min(p.V, x0 + p.chunk);
  const bool vec = (p.V & 3) == 0;
  const int g = p.host_map ? p.hgamma[i] : p.gamma[i];
  const int qst = p.host_map ? p.hq_start[i] : seq_start(p.gamma, i, sh), dst = qst - i;

  if (tid == 0) {
    sh.first_fail = g;
    sh.bad = 0;
  }
  __syncthreads();
  const bool greedy = p.mode == SV_ACCEPT_GREEDY;
  for (int j = tid; j < g; j += kThreads) {
    const int d = p.draft[dst + j];
    if (d < 0 || d >= p.V) {
      atomicOr(&sh.bad, 1);
    } else if (!greedy) {
      const float lhs = p.u_acc[dst + j] * p.q[(size_t)(dst + j) * p.V + d];
      const float pd = pxf_of(p, qst + j)(p.p[(size_t)(qst + j) * p.V + d]);
      if (!(lhs < pd)) atomicMin(&sh.first_fail, j);
    }
  }
  __syncthreads();
  const bool bad = sh.bad != 0;

  if (greedy) {
    // chunk argmax of each target row of the sequence
    if (!bad) {
      for (int j = 0; j <= g; ++j) {
        float bv;
        int bi;
        chunk_argmax(p.p + (size_t)(qst + j) * p.V, pxf_of(p, qst + j), x0, x1, vec, bv, bi);
        u64 z0 = 0, z1 = 0;
        block_reduce(z0, z1, bv, bi, sh);
        if (tid == 0) put_part(p.parts + (size_t)(qst + j) * p.nchunk + c, 0ull, 0ull, bv, bi);
      }
    }
    if (!arrive_last(p.counters + i, p.nchunk, sh)) return;
    if (bad) {
      if (tid == 0) commit_bad(p, i);
      return;
    }
    // leading drafts equal to their row's argmax, then that row's argmax
    int a = g, y = -1;
    for (int j = 0; j <= g; ++j) {
      float v = -INFINITY;
      int ix = 0x7fffffff;
      for (int cc = tid; cc < p.nchunk; cc += kThreads) {
        const AcceptPart q = get_part(p.parts + (size_t)(qst + j) * p.nchunk + cc);
        amax(v, ix, q.max_p, q.arg_p);
      }
      u64 z0 = 0, z1 = 0;
      block_reduce(z0, z1, v, ix, sh);
      if (j < g && p.draft[dst + j] == ix) continue;
      a = j;
      y = ix;
      break;
    }
    if (tid == 0) {
      p.accepted[i] = a;
      p.next_token[i] = y;
      p.kv_len[i] += a + 1;
    }
    return;
  }

  // ---- stochastic -----------------------------------------------------------
  const int a = sh.first_fail;
  const float *prow = p.p + (size_t)(qst + a) * p.V;
  const PXf xf = pxf_of(p, qst + a);
  const float *qrow = a < g ? p.q + (size_t)(dst + a) * p.V : nullptr;
  u64 sres = 0, sp = 0;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (!bad) {
    if (vec) {
      // all of this thread's loads first (kVecA float4 of each row), then the sums
      const float4 *p4 = reinterpret_cast<const float4 *>(prow);
      const float4 *q4 = reinterpret_cast<const float4 *>(qrow);
      float4 pv[kVecA], qv[kVecA];
#pragma unroll
      for (int k = 0; k < kVecA; ++k) {
        const int x = x0 / 4 + tid + k * kThreads;
        pv[k] = x < x1 / 4 ? xf(p4[x]) : make_float4(0.f, 0.f, 0.f, 0.f);
        qv[k] = (qrow && x < x1 / 4) ? q4[x] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < kVecA; ++k) {
        const int x = x0 / 4 + tid + k * kThreads;
        if (x >= x1 / 4) continue;
        const float pe[4] = {pv[k].x, pv[k].y, pv[k].z, pv[k].w};
        const float qe[4] = {qv[k].x, qv[k].y, qv[k].z, qv[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const u64 w = weight_of(pe[e]);
          sres += qrow ? weight_of(pe[e] - qe[e]) : w;
          sp += w;
          amax(bv, bi, pe[e], 4 * x + e);
        }
      }
    } else {
      for (int x = x0 + tid; x < x1; x += kThreads) {
        const float pv = xf(prow[x]);
        const u64 w = weight_of(pv);
        sres += qrow ? weight_of(pv - qrow[x]) : w;
        sp += w;
        amax(bv, bi, pv, x);
      }
    }
  }
  block_reduce(sres, sp, bv, bi, sh);
  if (tid == 0) put_part(p.parts + (size_t)i * p.nchunk + c, sres, sp, bv, bi);
  if (!arrive_last(p.counters + i, p.nchunk, sh)) return;
  if (bad) {
    if (tid == 0) commit_bad(p, i);
    return;
  }

  // totals over the chunks (chunk results staged in LDS once when they fit)
  const AcceptPart *pp = p.parts + (size_t)i * p.nchunk;
  __shared__ AcceptPart cpart[kThreads];
  const bool staged = p.nchunk <= kThreads;
  if (staged) {
    if (tid < p.nchunk) cpart[tid] = get_part(pp + tid);
    __syncthreads();
  }
  u64 s_res = 0, s_p = 0;
  float mv = -INFINITY;
  int mi = 0x7fffffff;
  for (int cc = tid; cc < p.nchunk; cc += kThreads) {
    const AcceptPart q = staged ? cpart[cc] : get_part(pp + cc);
    s_res += q.sum_res;
    s_p += q.sum_p;
    amax(mv, mi, q.max_p, q.arg_p);
  }
  block_reduce(s_res, s_p, mv, mi, sh);
  // weights: the resampling row, else the target row, else the argmax
  const int ur = s_res > 0 ? 1 : (s_p > 0 ? 0 : -1);
  int result = mi;
  if (ur >= 0) {
    const u64 S = ur ? s_res : s_p;
    u64 t = static_cast<u64>(floor(static_cast<double>(p.u_samp[i]) * static_cast<double>(S)));
    if (t >= S) t = S - 1;
    // the chunk holding t: scan the chunk sums in thread order, 256 at a time
    if (tid == 0) {
      sh.found = 0;
      sh.chunk_hit = p.nchunk - 1;
      sh.target = 0;
    }
    __syncthreads();
    u64 run = 0;
    for (int base = 0; base < p.nchunk; base += kThreads) {
      const int cc = base + tid;
      u64 v = 0;
      if (cc < p.nchunk) {
        const AcceptPart q = staged ? cpart[cc] : get_part(pp + cc);
        v = ur ? q.sum_res : q.sum_p;
      }
      u64 tot;
      const u64 before = run + block_exscan(v, &tot, sh);
      if (v > 0 && before <= t && t < before + v) {
        sh.found = 1;
        sh.chunk_hit = cc;
        sh.target = t - before;
      }
      run += tot;
      __syncthreads();
      if (sh.found) break;
    }
    // exact scan of that chunk: each thread a contiguous segment of `per`
    // elements (16-byte loads when rows are 16-byte aligned)
    const int cx0 = sh.chunk_hit * p.chunk, cx1 = min(p.V, cx0 + p.chunk);
    const int n = cx1 - cx0;
    const bool resid = ur == 1 && a < g;
    int per = (n + kThreads - 1) / kThreads;  // <= kSegMax
    if (vec) per = (per + 3) & ~3;             // whole float4s (n is a multiple of 4)
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    float wv[kSegMax];
    u64 s = 0;
    if (vec) {
      const float4 *p4 = reinterpret_cast<const float4 *>(prow + cx0 + lo);
      const float4 *q4 = reinterpret_cast<const float4 *>(resid ? qrow + cx0 + lo : prow);
      const int n4 = (hi - lo) / 4;  // hi - lo is a multiple of 4 (n % 4 == 0 here)
      float4 pv[kSegMax / 4], qv[kSegMax / 4];
#pragma unroll
      for (int k = 0; k < kSegMax / 4; ++k) {
        pv[k] = k < n4 ? xf(p4[k]) : make_float4(0.f, 0.f, 0.f, 0.f);
        qv[k] = (resid && k < n4) ? q4[k] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < kSegMax / 4; ++k) {
        wv[4 * k] = pv[k].x - qv[k].x;
        wv[4 * k + 1] = pv[k].y - qv[k].y;
        wv[4 * k + 2] = pv[k].z - qv[k].z;
        wv[4 * k + 3] = pv[k].w - qv[k].w;
      }
#pragma unroll
      for (int k = 0; k < kSegMax; ++k) s += weight_of(wv[k]);
    } else {
#pragma unroll
      for (int k = 0; k < kSegMax; ++k) {
        const int x = lo + k;
        float r = 0.f;
        if (x < hi) r = resid ? xf(prow[cx0 + x]) - qrow[cx0 + x] : xf(prow[cx0 + x]);
        wv[k] = r;
        s += weight_of(r);
      }
    }
    u64 tot;
    const u64 before = block_exscan(s, &tot, sh);
    const u64 tt = sh.target;
    if (tid == 0) sh.result = -1;
    __syncthreads();
    if (s > 0 && before <= tt && tt < before + s) {
      u64 acc = before;
#pragma unroll
      for (int k = 0; k < kSegMax; ++k) {
        acc += weight_of(wv[k]);
        if (acc > tt) {
          sh.result = cx0 + lo + k;
          break;
        }
      }
    }
    __syncthreads();
    result = sh.result;
  }
  if (tid == 0) {
    p.accepted[i] = a;
    p.next_token[i] = result;
    p.kv_len[i] += a + 1;
  }
}

// Per-position acceptance counters: thread i takes sequence i; counts for
// positions 1..n_pos gather in LDS and each workgroup adds its totals to the
// caller's 64-bit counters (integer adds: the totals do not depend on order).
__global__ __launch_bounds__(kThreads) void position_counts_kernel(int B, int n_pos, const int *gamma,
                                                                   const int *accepted,
                                                                   unsigned long long *counts) {
  __shared__ unsigned int hist[2 * kMaxCountPositions];
  for (int k = threadIdx.x; k < 2 * n_pos; k += kThreads) hist[k] = 0;
  __syncthreads();
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < B) {
    const int a = accepted[i], g = gamma[i];
    if (a >= 0) {
      // draft k was tested iff k <= gamma_i and drafts 1..k-1 passed (k <= a + 1)
      const int reached = min(min(g, a + 1), n_pos), acc = min(a, n_pos);
      for (int k = 0; k < reached; ++k) atomicAdd(&hist[k], 1u);
      for (int k = 0; k < acc; ++k) atomicAdd(&hist[n_pos + k], 1u);
    }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < 2 * n_pos; k += kThreads)
    if (hist[k]) atomicAdd(&counts[k], (unsigned long long)hist[k]);
}

}  // namespace

hipError_t launch_position_counts(int B, int n_pos, const int *gamma, const int *accepted,
                                  unsigned long long *counts, hipStream_t s) {
  if (n_pos < 1 || n_pos > kMaxCountPositions) return hipErrorInvalidValue;
  hipLaunchKernelGGL(position_counts_kernel, dim3((B + kThreads - 1) / kThreads), dim3(kThreads), 0, s, B, n_pos,
                     gamma, accepted, counts);
  return hipGetLastError();
}

hipError_t launch_accept(const AcceptParams &p, hipStream_t s) {
  if (p.chunk > kThreads * kSegMax) return hipErrorInvalidValue;
  trace_before(SV_K_ACCEPT, s);
  hipLaunchKernelGGL(accept_kernel, dim3(p.nchunk, p.B), dim3(kThreads), 0, s, p);
  trace_after(SV_K_ACCEPT, s);
  return hipGetLastError();
}

}  // namespace sv
