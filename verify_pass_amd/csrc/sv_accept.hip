// Acceptance, resampling and KV-length commit, gfx950.
//
// Rejection sampling in the sense of Leviathan, Kalman and Matias keeps the
// output distribution of plain decoding; the verifier keeps the drafts up to
// the first rejection and adds one token of its own.  Draws use integer
// weights R(x) = trunc(fl32(r(x) * 2^32)): sums of integers do not depend on
// the order in which lanes and workgroups add them, so the token drawn for a
// given uniform is the same on any grid shape.
//
// Kernel 1 (grid: vocabulary chunks x sequences, or x rows in greedy mode):
//   acceptance tests (one draft per lane, first rejection by LDS atomic min),
//   then per-chunk weight sums of the residual / bonus row, of the fallback
//   target row, and the chunk's argmax.
// Kernel 2 (grid: sequences): total weight, uniform -> integer target,
//   chunk search over the partial sums, exact scan inside the chunk, commit.
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
}

// q_start of every sequence (exclusive scan of gamma + 1) into qs[0..B).
__device__ inline void token_starts(const int *gamma, int B, int *qs, int *tmp) {
  for (int i = threadIdx.x; i < B; i += kThreads) qs[i] = gamma[i] + 1;
  __syncthreads();
  block_exscan(qs, B, tmp);
}

__global__ __launch_bounds__(kThreads) void accept_scan_kernel(AcceptParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ u64 sa[kThreads], sb[kThreads];
  __shared__ float sv[kThreads];
  __shared__ int si[kThreads];
  __shared__ int first_fail, bad;
  int *qs = reinterpret_cast<int *>(smem);
  int *tmp = qs + p.B + 1;
  const int tid = threadIdx.x, c = blockIdx.x;
  const int x0 = c * p.chunk, x1 = min(p.V, x0 + p.chunk);

  if (p.mode == SV_ACCEPT_GREEDY) {
    // one target row per blockIdx.y: chunk argmax only
    const int row = blockIdx.y;
    const float *pr = p.p + (size_t)row * p.V;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int x = x0 + tid; x < x1; x += kThreads) amax(bv, bi, pr[x], x);
    u64 z0 = 0, z1 = 0;
    block_reduce(z0, z1, bv, bi, sa, sb, sv, si);
    if (tid == 0) p.parts[(size_t)row * p.nchunk + c] = AcceptPart{0ull, 0ull, bv, bi};
    return;
  }

  const int i = blockIdx.y;
  token_starts(p.gamma, p.B, qs, tmp);
  const int g = p.gamma[i];
  const int qst = qs[i], dst = qst - i;
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
  if (bad) {
    if (c == 0 && tid == 0) p.acc_ws[i] = -1;
    return;
  }
  const int a = first_fail;
  if (c == 0 && tid == 0) p.acc_ws[i] = a;
  const float *prow = p.p + (size_t)(qst + a) * p.V;
  const float *qrow = a < g ? p.q + (size_t)(dst + a) * p.V : nullptr;
  u64 sres = 0, sp = 0;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (qrow) {
    for (int x = x0 + tid; x < x1; x += kThreads) {
      const float pv = prow[x];
      sres += weight_of(pv - qrow[x]);
      sp += weight_of(pv);
      amax(bv, bi, pv, x);
    }
  } else {
    for (int x = x0 + tid; x < x1; x += kThreads) {
      const float pv = prow[x];
      const u64 w = weight_of(pv);
      sres += w;
      sp += w;
      amax(bv, bi, pv, x);
    }
  }
  block_reduce(sres, sp, bv, bi, sa, sb, sv, si);
  if (tid == 0) p.parts[(size_t)i * p.nchunk + c] = AcceptPart{sres, sp, bv, bi};
}

__global__ __launch_bounds__(kThreads) void accept_select_kernel(AcceptParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ u64 seg[kThreads + 1];
  __shared__ int chosen_chunk, use_res, result;
  __shared__ u64 target;
  __shared__ int row_arg[64];
  int *qs = reinterpret_cast<int *>(smem);
  int *tmp = qs + p.B + 1;
  const int tid = threadIdx.x, i = blockIdx.x;
  token_starts(p.gamma, p.B, qs, tmp);
  const int g = p.gamma[i];
  const int qst = qs[i], dst = qst - i;

  if (p.mode == SV_ACCEPT_GREEDY) {
    // argmax of each of the g + 1 rows (chunks combined in fixed order)
    for (int j = tid; j <= g; j += kThreads) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      const AcceptPart *pp = p.parts + (size_t)(qst + j) * p.nchunk;
      for (int c = 0; c < p.nchunk; ++c) amax(bv, bi, pp[c].max_p, pp[c].arg_p);
      if (j < 64) row_arg[j] = bi;
      else p.acc_ws[p.B + (qst + j)] = bi;  // rare long drafts spill to workspace
    }
    __syncthreads();
    if (tid == 0) {
      auto arg = [&](int j) { return j < 64 ? row_arg[j] : p.acc_ws[p.B + qst + j]; };
      int a = 0, badtok = 0;
      for (int j = 0; j < g; ++j) {
        const int d = p.draft[dst + j];
        if (d < 0 || d >= p.V) { badtok = 1; break; }
      }
      if (badtok) {
        p.accepted[i] = -1;
        p.next_token[i] = -1;
        set_err(p.err, SV_DEV_ERR_BAD_TOKEN);
        return;
      }
      while (a < g && p.draft[dst + a] == arg(a)) ++a;
      p.accepted[i] = a;
      p.next_token[i] = arg(a);
      p.kv_len[i] += a + 1;
    }
    return;
  }

  const int a = p.acc_ws[i];
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
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int c = 0; c < p.nchunk; ++c) {
      s_res += pp[c].sum_res;
      s_p += pp[c].sum_p;
      amax(bv, bi, pp[c].max_p, pp[c].arg_p);
    }
    int ur;
    u64 S;
    if (s_res > 0) { ur = 1; S = s_res; }
    else if (s_p > 0) { ur = 0; S = s_p; }
    else { ur = -1; S = 0; }
    use_res = ur;
    result = -1;
    if (ur < 0) {
      result = bi;
    } else {
      u64 t = static_cast<u64>(floor(static_cast<double>(p.u_samp[i]) * static_cast<double>(S)));
      if (t >= S) t = S - 1;
      u64 run = 0;
      int cc = p.nchunk - 1;
      for (int c = 0; c < p.nchunk; ++c) {
        const u64 v = ur ? pp[c].sum_res : pp[c].sum_p;
        if (run + v > t) { cc = c; break; }
        run += v;
      }
      chosen_chunk = cc;
      target = t - run;
    }
  }
  __syncthreads();
  if (use_res >= 0) {
    const int c = chosen_chunk;
    const int x0 = c * p.chunk, x1 = min(p.V, x0 + p.chunk);
    const int n = x1 - x0;
    const int per = (n + kThreads - 1) / kThreads;
    const int lo = x0 + min(n, tid * per), hi = x0 + min(n, (tid + 1) * per);
    const float *prow = p.p + (size_t)(qst + a) * p.V;
    const float *qrow = (use_res && a < g) ? p.q + (size_t)(dst + a) * p.V : nullptr;
    u64 s = 0;
    for (int x = lo; x < hi; ++x) s += weight_of(qrow ? prow[x] - qrow[x] : prow[x]);
    seg[tid] = s;
    __syncthreads();
    if (tid == 0) {
      u64 run = 0;
      for (int k = 0; k < kThreads; ++k) {
        const u64 v = seg[k];
        seg[k] = run;
        run += v;
      }
      seg[kThreads] = run;
    }
    __syncthreads();
    const u64 t = target;
    const u64 before = seg[tid];
    if (before <= t && t < before + s) {
      u64 run = before;
      for (int x = lo; x < hi; ++x) {
        run += weight_of(qrow ? prow[x] - qrow[x] : prow[x]);
        if (run > t) { result = x; break; }
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
  const size_t lds = (size_t)(p.B + 1 + 260) * sizeof(int);
  const int rows = p.mode == SV_ACCEPT_GREEDY ? p.T : p.B;
  trace_before(SV_K_ACCEPT_SCAN, s);
  hipLaunchKernelGGL(accept_scan_kernel, dim3(p.nchunk, rows), dim3(kThreads), lds, s, p);
  trace_after(SV_K_ACCEPT_SCAN, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  trace_before(SV_K_ACCEPT_SELECT, s);
  hipLaunchKernelGGL(accept_select_kernel, dim3(p.B), dim3(kThreads), lds, s, p);
  trace_after(SV_K_ACCEPT_SELECT, s);
  return hipGetLastError();
}

}  // namespace sv
