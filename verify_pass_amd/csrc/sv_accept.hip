// Acceptance, resampling and KV-length commit, gfx950.
//
// Rejection sampling in the sense of Leviathan, Kalman and Matias keeps the
// output distribution of plain decoding; the verifier keeps the drafts up to
// the first rejection and adds one token of its own.  Draws use integer
// weights R(x) = trunc(fl32(r(x) * 2^32)): sums of integers do not depend on
// the order in which lanes and workgroups add them, so the token drawn for a
// given uniform is the same on any grid shape.
//
// One kernel, grid = vocabulary chunks x sequences (x target rows in greedy
// mode).  Every workgroup runs the sequence's acceptance tests (one draft per
// lane, first rejection by LDS atomic min) and sums the integer weights of its
// chunk of the resampling row, of the fallback target row, and the chunk's
// argmax.  It publishes them with device-scope stores and bumps the
// sequence's arrival counter; the last workgroup to arrive turns the uniform
// into an integer target, finds the chunk holding it from the chunk sums,
// scans that chunk exactly (staged through LDS) and commits.
#include "sv_common.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr float kTwo32 = 4294967296.0f;

typedef unsigned long long u64;

__device__ __forceinline__ u64 weight_of(float r) {
  r = fmaxf(r, 0.f);
  return static_cast<u64>(r * kTwo32);
}

// argmax combine: larger value wins, lower index on ties
__device__ __forceinline__ void amax(float &v, int &i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

__device__ inline void block_reduce(u64 &a, u64 &b, float &v, int &ix, u64 *sa, u64 *sb, float *sv,
                                    int *si) {
  const int tid = threadIdx.x;
  sa[tid] = a;
  sb[tid] = b;
  sv[tid] = v;
  si[tid] = ix;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (tid < o) {
      sa[tid] += sa[tid + o];
      sb[tid] += sb[tid + o];
      float vv = sv[tid];
      int ii = si[tid];
      amax(vv, ii, sv[tid + o], si[tid + o]);
      sv[tid] = vv;
      si[tid] = ii;
    }
    __syncthreads();
  }
  a = sa[0];
  b = sb[0];
  v = sv[0];
  ix = si[0];
  __syncthreads();
}

// Device-scope (cross-XCD coherent) stores and loads of the chunk results.
__device__ __forceinline__ void put_part(AcceptPart *p, const AcceptPart &v) {
  u64 *w = reinterpret_cast<u64 *>(p);
  __hip_atomic_store(w, v.sum_res, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(w + 1, v.sum_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const u64 mx = (static_cast<u64>(static_cast<uint32_t>(v.arg_p)) << 32) | __float_as_uint(v.max_p);
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

// Publish, count the arrival, and tell whether this workgroup arrived last
// (then the counter is reset for the next call).
__device__ inline bool arrive_last(int *ctr, int expected, int *flag) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = old == expected - 1;
    if (*flag) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *flag != 0;
}

// q_start of sequence i (exclusive prefix sum of gamma + 1), by a block reduction.
__device__ inline int seq_start(const int *gamma, int i, int *red) {
  int s = 0;
  for (int k = threadIdx.x; k < i; k += kThreads) s += gamma[k] + 1;
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const int r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void accept_kernel(AcceptParams p) {
  __shared__ u64 sa[kThreads], sb[kThreads];
  __shared__ float sv[kThreads];
  __shared__ int si[kThreads];
  __shared__ int red[kThreads];
  __shared__ int first_fail, bad, flag, chosen_chunk, use_res, result;
  __shared__ u64 target, seg[kThreads];
  __shared__ int row_arg[64];
  __shared__ float stage_p[8192];
  __shared__ float stage_q[8192];
  const int tid = threadIdx.x, c = blockIdx.x;
  const int x0 = c * p.chunk, x1 = min(p.V, x0 + p.chunk);

  if (p.mode == SV_ACCEPT_GREEDY) {
    // blockIdx.y = target row: chunk argmax; the last of the sequence's
    // (gamma_i + 1) * nchunk workgroups decides
    const int row = blockIdx.y;
    const float *pr = p.p + (size_t)row * p.V;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int x = x0 + tid; x < x1; x += kThreads) amax(bv, bi, pr[x], x);
    u64 z0 = 0, z1 = 0;
    block_reduce(z0, z1, bv, bi, sa, sb, sv, si);
    if (tid == 0) put_part(p.parts + (size_t)row * p.nchunk + c, AcceptPart{0ull, 0ull, bv, bi});
    // owner sequence of this row
    if (tid == 0) {
      int s = 0, i = 0;
      while (i < p.B && s + p.gamma[i] + 1 <= row) s += p.gamma[i++] + 1;
      red[0] = i;
      red[1] = s;
    }
    __syncthreads();
    const int i = red[0], qst = red[1];
    __syncthreads();
    const int g = p.gamma[i];
    if (!arrive_last(p.counters + i, (g + 1) * p.nchunk, &flag)) return;
    for (int j = tid; j <= g; j += kThreads) {
      float v = -INFINITY;
      int b = 0x7fffffff;
      for (int cc = 0; cc < p.nchunk; ++cc) {
        const AcceptPart q = get_part(p.parts + (size_t)(qst + j) * p.nchunk + cc);
        amax(v, b, q.max_p, q.arg_p);
      }
      if (j < 64) row_arg[j] = b;
      else p.acc_ws[p.B + qst + j] = b;  // rare long drafts spill to workspace
    }
    wait_vmem();
    __syncthreads();
    if (tid == 0) {
      const int dst = qst - i;
      auto arg = [&](int j) {
        return j < 64 ? row_arg[j]
                      : __hip_atomic_load(p.acc_ws + p.B + qst + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      };
      int badtok = 0;
      for (int j = 0; j < g; ++j) {
        const int d = p.draft[dst + j];
        if (d < 0 || d >= p.V) badtok = 1;
      }
      if (badtok) {
        p.accepted[i] = -1;
        p.next_token[i] = -1;
        set_err(p.err, SV_DEV_ERR_BAD_TOKEN);
        return;
      }
      int a = 0;
      while (a < g && p.draft[dst + a] == arg(a)) ++a;
      p.accepted[i] = a;
      p.next_token[i] = arg(a);
      p.kv_len[i] += a + 1;
    }
    return;
  }

  // ---- stochastic -----------------------------------------------------------
  const int i = blockIdx.y;
  const int g = p.gamma[i];
  const int qst = seq_start(p.gamma, i, red), dst = qst - i;
  if (tid == 0) {
    first_fail = g;
    bad = 0;
  }
  __syncthreads();
  for (int j = tid; j < g; j += kThreads) {
    const int d = p.draft[dst + j];
    if (d < 0 || d >= p.V) {
      atomicOr(&bad, 1);
    } else {
      const float lhs = p.u_acc[dst + j] * p.q[(size_t)(dst + j) * p.V + d];
      if (!(lhs < p.p[(size_t)(qst + j) * p.V + d])) atomicMin(&first_fail, j);
    }
  }
  __syncthreads();
  const int a = bad ? -1 : first_fail;
  const float *prow = p.p + (size_t)(qst + max(a, 0)) * p.V;
  const float *qrow = (a >= 0 && a < g) ? p.q + (size_t)(dst + a) * p.V : nullptr;
  u64 sres = 0, sp = 0;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (a >= 0) {
    for (int x = x0 + tid; x < x1; x += kThreads) {
      const float pv = prow[x];
      const u64 w = weight_of(pv);
      sres += qrow ? weight_of(pv - qrow[x]) : w;
      sp += w;
      amax(bv, bi, pv, x);
    }
  }
  block_reduce(sres, sp, bv, bi, sa, sb, sv, si);
  if (tid == 0) put_part(p.parts + (size_t)i * p.nchunk + c, AcceptPart{sres, sp, bv, bi});
  if (!arrive_last(p.counters + i, p.nchunk, &flag)) return;

  if (a < 0) {
    if (tid == 0) {
      p.accepted[i] = -1;
      p.next_token[i] = -1;
      set_err(p.err, SV_DEV_ERR_BAD_TOKEN);
    }
    return;
  }
  const AcceptPart *pp = p.parts + (size_t)i * p.nchunk;
  if (tid == 0) {
    u64 s_res = 0, s_p = 0;
    float mv = -INFINITY;
    int mi = 0x7fffffff;
    for (int cc = 0; cc < p.nchunk; ++cc) {
      const AcceptPart q = get_part(pp + cc);
      s_res += q.sum_res;
      s_p += q.sum_p;
      amax(mv, mi, q.max_p, q.arg_p);
    }
    int ur;
    u64 S;
    if (s_res > 0) { ur = 1; S = s_res; }
    else if (s_p > 0) { ur = 0; S = s_p; }
    else { ur = -1; S = 0; }
    use_res = ur;
    result = -1;
    if (ur < 0) {
      result = mi;
    } else {
      u64 t = static_cast<u64>(floor(static_cast<double>(p.u_samp[i]) * static_cast<double>(S)));
      if (t >= S) t = S - 1;
      u64 run = 0;
      int cc_hit = p.nchunk - 1;
      for (int cc = 0; cc < p.nchunk; ++cc) {
        const AcceptPart q = get_part(pp + cc);
        const u64 v = ur ? q.sum_res : q.sum_p;
        if (run + v > t) { cc_hit = cc; break; }
        run += v;
      }
      chosen_chunk = cc_hit;
      target = t - run;
    }
  }
  __syncthreads();
  if (use_res >= 0) {
    // exact scan of the chosen chunk: stage it in LDS with coalesced loads,
    // then each thread sums a contiguous segment
    const int cx0 = chosen_chunk * p.chunk, cx1 = min(p.V, cx0 + p.chunk);
    const int n = cx1 - cx0;
    const bool resid = use_res && a < g;
    for (int x = tid; x < n; x += kThreads) {
      stage_p[x] = prow[cx0 + x];
      if (resid) stage_q[x] = qrow[cx0 + x];
    }
    __syncthreads();
    const int per = (n + kThreads - 1) / kThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    u64 s = 0;
    for (int x = lo; x < hi; ++x) s += weight_of(resid ? stage_p[x] - stage_q[x] : stage_p[x]);
    seg[tid] = s;
    __syncthreads();
    if (tid == 0) {
      u64 run = 0;
      for (int k = 0; k < kThreads; ++k) {
        const u64 v = seg[k];
        seg[k] = run;
        run += v;
      }
    }
    __syncthreads();
    const u64 t = target, before = seg[tid];
    if (before <= t && t < before + s) {
      u64 run = before;
      for (int x = lo; x < hi; ++x) {
        run += weight_of(resid ? stage_p[x] - stage_q[x] : stage_p[x]);
        if (run > t) { result = cx0 + x; break; }
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    p.accepted[i] = a;
    p.next_token[i] = result;
    p.kv_len[i] += a + 1;
  }
}

}  // namespace

hipError_t launch_accept(const AcceptParams &p, hipStream_t s) {
  const int rows = p.mode == SV_ACCEPT_GREEDY ? p.T : p.B;
  trace_before(SV_K_ACCEPT, s);
  hipLaunchKernelGGL(accept_kernel, dim3(p.nchunk, rows), dim3(kThreads), 0, s, p);
  trace_after(SV_K_ACCEPT, s);
  return hipGetLastError();
}

}  // namespace sv
