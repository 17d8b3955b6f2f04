// Token-tree acceptance and the commit's cache-row moves, gfx950.
//
// One workgroup walks one sequence's tree from the root.  At a node v the
// children are tested in index order: the first by the linear rule
// (fl32(u * q_v(d)) < p_v(d)); after a rejection the target becomes the
// integer residual R of the rejected candidates (first R(x) =
// trunc(fl32(max(0, fl32(p_v(x) - q_v(x))) * 2^32)), S = sum R), a later
// sibling d passes iff U * Q(d) * S < R(d) * SQ * 2^24 (U = u * 2^24,
// Q(x) = trunc(fl32(q_v(x) * 2^32)), SQ = sum Q), and each further rejection
// replaces R by max(0, R * SQ - Q * S) shifted right until its sum fits 32
// bits.  The first passing child becomes v; with none (or at a leaf) the
// token is drawn from R (or from trunc(fl32(p_v * 2^32)), the bonus row) by
// the integer inverse CDF.  Every decision is exact integer arithmetic or one
// fp32 compare, so any thread layout decides the same.  Greedy mode follows
// the child whose token is argmax p_v.
//
// The commit then moves each accepted node's key and value from cache row
// ctx + node to ctx + depth, in increasing depth (a node's index is at least
// its depth, so no move reads a row an earlier move wrote).
#include "sv_common.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr float kTwo32 = 4294967296.0f;
typedef unsigned long long u64;

__device__ __forceinline__ u64 weight_of(float r) { return static_cast<u64>(fmaxf(r, 0.f) * kTwo32); }

// Unsigned 128-bit values as (hi, lo) pairs.
struct U128 {
  u64 hi, lo;
};
__device__ __forceinline__ U128 mul64(u64 a, u64 b) { return U128{__umul64hi(a, b), a * b}; }
__device__ __forceinline__ U128 add128(U128 a, U128 b) {
  const u64 lo = a.lo + b.lo;
  return U128{a.hi + b.hi + (lo < a.lo ? 1ull : 0ull), lo};
}
__device__ __forceinline__ bool less128(U128 a, U128 b) { return a.hi < b.hi || (a.hi == b.hi && a.lo < b.lo); }
// max(0, a - b)
__device__ __forceinline__ U128 subsat128(U128 a, U128 b) {
  if (less128(a, b)) return U128{0ull, 0ull};
  return U128{a.hi - b.hi - (a.lo < b.lo ? 1ull : 0ull), a.lo - b.lo};
}
__device__ __forceinline__ U128 shl128(U128 a, int s) {  // 0 < s < 64
  return U128{(a.hi << s) | (a.lo >> (64 - s)), a.lo << s};
}
__device__ __forceinline__ u64 shr128_lo(U128 a, int s) {  // low word of a >> s, 0 <= s < 128
  if (s == 0) return a.lo;
  if (s >= 64) return a.hi >> (s - 64);
  return (a.lo >> s) | (a.hi << (64 - s));
}
__device__ __forceinline__ int bitlen128(U128 a) {
  return a.hi ? 128 - __clzll(a.hi) : (a.lo ? 64 - __clzll(a.lo) : 0);
}

struct TreeShared {
  int par[kMaxTreeNodes];
  int tok[kMaxTreeNodes];
  int path[kMaxTreeNodes];
  int bad;
  int cur, next_child, ok, result;
  u64 s64;
  U128 s128;
  u64 red64[kThreads];
  U128 red128[kThreads];
  float amax_v[kThreads];
  int amax_i[kThreads];
};

__device__ u64 block_sum64(u64 v, TreeShared &sh) {
  const int tid = threadIdx.x;
  sh.red64[tid] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (tid < s) sh.red64[tid] += sh.red64[tid + s];
    __syncthreads();
  }
  const u64 r = sh.red64[0];
  __syncthreads();
  return r;
}

__device__ U128 block_sum128(U128 v, TreeShared &sh) {
  const int tid = threadIdx.x;
  sh.red128[tid] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (tid < s) sh.red128[tid] = add128(sh.red128[tid], sh.red128[tid + s]);
    __syncthreads();
  }
  const U128 r = sh.red128[0];
  __syncthreads();
  return r;
}

// argmax of row[0, V), lowest index on ties
__device__ int block_argmax(const float *row, int V, TreeShared &sh) {
  const int tid = threadIdx.x;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int x = tid; x < V; x += kThreads) {
    const float v = row[x];
    if (v > bv || (v == bv && x < bi)) {
      bv = v;
      bi = x;
    }
  }
  sh.amax_v[tid] = bv;
  sh.amax_i[tid] = bi;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
      const float v2 = sh.amax_v[tid + s];
      const int i2 = sh.amax_i[tid + s];
      if (v2 > sh.amax_v[tid] || (v2 == sh.amax_v[tid] && i2 < sh.amax_i[tid])) {
        sh.amax_v[tid] = v2;
        sh.amax_i[tid] = i2;
      }
    }
    __syncthreads();
  }
  const int r = sh.amax_i[0] == 0x7FFFFFFF ? 0 : sh.amax_i[0];
  __syncthreads();
  return r;
}

// The least x whose running sum of R exceeds t (t < sum R): each thread owns
// one contiguous segment; segment sums are scanned in thread order.
__device__ int block_draw(const u64 *R, int V, u64 t, TreeShared &sh) {
  const int tid = threadIdx.x;
  const int per = (V + kThreads - 1) / kThreads;
  const int x0 = min(V, tid * per), x1 = min(V, x0 + per);
  u64 seg = 0;
  for (int x = x0; x < x1; ++x) seg += R[x];
  sh.red64[tid] = seg;
  if (tid == 0) sh.result = V - 1;  // (t < sum R: some segment holds it)
  __syncthreads();
  if (tid == 0) {
    u64 run = 0;
    for (int k = 0; k < kThreads; ++k) {
      const u64 v = sh.red64[k];
      sh.red64[k] = run;
      run += v;
    }
  }
  __syncthreads();
  const u64 before = sh.red64[tid];
  if (t >= before && t < before + seg) {
    u64 run = before;
    for (int x = x0; x < x1; ++x) {
      run += R[x];
      if (run > t) {
        sh.result = x;
        break;
      }
    }
  }
  __syncthreads();
  const int r = sh.result;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void tree_accept_kernel(TreeAcceptParams p) {
  __shared__ TreeShared sh;
  const int i = blockIdx.x, tid = threadIdx.x;
  const int qs = p.q_start[i], n = p.q_start[i + 1] - qs;
  const int V = p.V;
  u64 *R = p.rbuf + (size_t)i * V;
  if (tid == 0) sh.bad = 0;
  __syncthreads();
  for (int j = tid; j < n; j += kThreads) {
    const int pj = p.parent[qs + j], tj = p.tokens[qs + j];
    sh.par[j] = pj;
    sh.tok[j] = tj;
    if (j > 0 && (pj < 0 || pj >= j)) atomicOr(&sh.bad, SV_DEV_ERR_BAD_TREE);
    if (j > 0 && (tj < 0 || tj >= V)) atomicOr(&sh.bad, SV_DEV_ERR_BAD_TOKEN);
  }
  __syncthreads();
  if (sh.bad) {
    if (tid == 0) {
      set_err(p.err, sh.bad);
      p.accepted[i] = -1;
      p.next_token[i] = -1;
      for (int k = 0; k < kMaxTreeNodes; ++k) p.path[(size_t)i * kMaxTreeNodes + k] = -1;
    }
    return;
  }
  int v = 0, depth = 0, y = 0;
  if (tid == 0) sh.path[0] = 0;
  for (;;) {
    const float *pv = p.p + (size_t)(qs + v) * V;
    if (p.greedy) {
      const int am = block_argmax(pv, V, sh);
      if (tid == 0) {
        sh.next_child = -1;
        for (int c = v + 1; c < n; ++c)
          if (sh.par[c] == v && sh.tok[c] == am) {
            sh.next_child = c;
            break;
          }
      }
      __syncthreads();
      const int c = sh.next_child;
      __syncthreads();
      if (c < 0) {
        y = am;
        break;
      }
      v = c;
      ++depth;
      if (tid == 0) sh.path[depth] = c;
      continue;
    }
    const float *qv = p.q + (size_t)(qs + v) * V;
    bool have_r = false;  // R holds the residual of the rejected children
    u64 S = 0, SQ = 0;
    bool sq_ready = false;
    int moved = -1;
    for (int c = v + 1; c < n; ++c) {
      if (sh.par[c] != v) continue;  // same value on every thread (LDS)
      const int d = sh.tok[c];
      if (!have_r) {
        if (tid == 0) sh.ok = (p.u_acc[qs + c] * qv[d] < pv[d]) ? 1 : 0;
      } else {
        if (!sq_ready) {
          u64 part = 0;
          for (int x = tid; x < V; x += kThreads) part += weight_of(qv[x]);
          SQ = block_sum64(part, sh);
          sq_ready = true;
        }
        if (tid == 0) {
          const u64 U = static_cast<u64>(static_cast<double>(p.u_acc[qs + c]) * 16777216.0);
          const U128 lhs = mul64(U * weight_of(qv[d]), S);
          const U128 rhs = shl128(mul64(R[d], SQ), 24);
          sh.ok = less128(lhs, rhs) ? 1 : 0;
        }
      }
      __syncthreads();
      const int ok = sh.ok;
      __syncthreads();
      if (ok) {
        moved = c;
        break;
      }
      // rejected: the residual becomes the target
      if (!have_r) {
        u64 part = 0;
        for (int x = tid; x < V; x += kThreads) {
          const u64 w = weight_of(pv[x] - qv[x]);
          R[x] = w;
          part += w;
        }
        S = block_sum64(part, sh);
        have_r = true;
      } else {
        U128 part{0ull, 0ull};
        for (int x = tid; x < V; x += kThreads)
          part = add128(part, subsat128(mul64(R[x], SQ), mul64(weight_of(qv[x]), S)));
        const U128 tot = block_sum128(part, sh);
        const int shift = max(0, bitlen128(tot) - 32);
        // every thread rewrites only the entries it read
        u64 part2 = 0;
        for (int x = tid; x < V; x += kThreads) {
          const u64 w = shr128_lo(subsat128(mul64(R[x], SQ), mul64(weight_of(qv[x]), S)), shift);
          R[x] = w;
          part2 += w;
        }
        S = block_sum64(part2, sh);
      }
      if (S == 0) {  // empty residual: back to the target row
        u64 part = 0;
        for (int x = tid; x < V; x += kThreads) {
          const u64 w = weight_of(pv[x]);
          R[x] = w;
          part += w;
        }
        S = block_sum64(part, sh);
      }
    }
    if (moved >= 0) {
      v = moved;
      ++depth;
      if (tid == 0) sh.path[depth] = moved;
      continue;
    }
    // draw: the residual after rejections, or the bonus row p_v
    if (!have_r) {
      u64 part = 0;
      for (int x = tid; x < V; x += kThreads) {
        const u64 w = weight_of(pv[x]);
        R[x] = w;
        part += w;
      }
      S = block_sum64(part, sh);
    }
    __syncthreads();  // R complete before the segment scan reads it
    if (S == 0) {
      y = block_argmax(pv, V, sh);
    } else {
      u64 t = static_cast<u64>(floor(static_cast<double>(p.u_samp[i]) * static_cast<double>(S)));
      if (t > S - 1) t = S - 1;
      y = block_draw(R, V, t, sh);
    }
    break;
  }
  __syncthreads();
  if (tid == 0) {
    p.accepted[i] = depth;
    p.next_token[i] = y;
    p.kv_len[i] += depth + 1;
  }
  for (int k = tid; k < kMaxTreeNodes; k += kThreads)
    p.path[(size_t)i * kMaxTreeNodes + k] = k <= depth ? sh.path[k] : -1;
}

// Row moves of the commit, one workgroup per (sequence, KV head).
__global__ __launch_bounds__(kThreads) void tree_commit_kernel(TreeCommitParams p) {
  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int a = p.accepted[i];
  if (a <= 0) return;
  const int ctx = p.kv_len[i] - a - 1;
  const int *path = p.path + (size_t)i * kMaxTreeNodes;
  uint16_t *kc = static_cast<uint16_t *>(p.kc[i]) + (size_t)h * p.kv_cap * p.hd;
  uint16_t *vc = static_cast<uint16_t *>(p.vc[i]) + (size_t)h * p.hd * p.kv_cap;
  for (int k = 1; k <= a && k < kMaxTreeNodes; ++k) {
    const int node = path[k];
    const int src = ctx + node, dst = ctx + k;
    const bool move = node > k && node < kMaxTreeNodes && ctx >= 0 && src < p.kv_cap;
    if (move) {
      for (int c = tid; c < p.hd; c += kThreads) {
        kc[(size_t)dst * p.hd + c] = kc[(size_t)src * p.hd + c];
        // values in 32-position blocks: (position, column) at (pos / 32 * hd + column) * 32 + pos % 32
        vc[((size_t)(dst >> 5) * p.hd + c) * 32 + (dst & 31)] = vc[((size_t)(src >> 5) * p.hd + c) * 32 + (src & 31)];
      }
    }
    __syncthreads();  // depth k lands before depth k + 1 reads
  }
}

}  // namespace

hipError_t launch_tree_accept(const TreeAcceptParams &p, hipStream_t s) {
  trace_before(SV_K_ACCEPT, s);
  hipLaunchKernelGGL(tree_accept_kernel, dim3(p.B), dim3(kThreads), 0, s, p);
  trace_after(SV_K_ACCEPT, s);
  return hipGetLastError();
}

hipError_t launch_tree_commit(const TreeCommitParams &p, hipStream_t s) {
  hipLaunchKernelGGL(tree_commit_kernel, dim3(p.B, p.hkv), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
