// Token-tree acceptance and the commit's cache-row moves, gfx950.
//
// The walk goes down from the root.  At a node v the children are tested in
// index order: the first by the linear rule (fl32(u * q_v(d)) < p_v(d));
// after a rejection the target becomes the integer residual R of the
// rejected candidates (first R(x) = trunc(fl32(max(0, fl32(p_v(x) - q_v(x)))
// * 2^32)), S = sum R, with R = trunc(fl32(p_v * 2^32)) when that sum is 0),
// a later sibling d passes iff U * Q(d) * S < R(d) * SQ * 2^24 (U = u * 2^24,
// Q(x) = trunc(fl32(q_v(x) * 2^32)), SQ = sum Q), and each further rejection
// replaces R by max(0, R * SQ - Q * S) shifted right until its sum fits 32
// bits.  The first passing child becomes v; with none (or at a leaf) the
// token is drawn from R (or from trunc(fl32(p_v * 2^32)), the bonus row) by
// the integer inverse CDF.  Every decision is exact integer arithmetic or one
// fp32 compare, so any thread and workgroup layout decides the same.  Greedy
// mode follows the child whose token is argmax p_v.  The target rows may be
// logits with each row's (max, sum of exponentials): every entry read is then
// turned into the probability the head's softmax finish would have written.
//
// The walk itself touches a few entries per node; what costs is the
// vocabulary-long sums behind a rejection and the draw.  Those run on grids
// of vocabulary chunks (4096 entries, one workgroup each).  Stochastic mode,
// six launches:
//   walk 1 (sequences): one workgroup per tree gathers every node's own test
//          inputs once and walks down in LDS.  It ends on a draw from p_v (a
//          leaf) or from the first residual (the only child rejected), or
//          stops where a rejected first child has a sibling: that test needs
//          sum Q and the first residual's sum;
//   sums   (chunks x nodes): per chunk, sum w(p), sum w(p - q), sum w(q) of
//          the nodes walk 1 flagged: the stopping node and those of two or
//          more children below its second child;
//   walk 2 (sequences): the stopped walks go on from the chunk totals and end
//          on a draw from p_v, the first or the second residual (both of two
//          children rejected).  A node that needs sums it does not have, or a
//          third sibling's test (it needs the second residual's sum), is
//          finished by the workgroup alone, with the residual in its own [V]
//          buffer;
//   resid2 (chunks x sequences): the 128-bit chunk sums of the unshifted
//          second residual, whose total fixes the shift;
//   draw   (chunks x sequences): per chunk, the sum of the draw's weights, of
//          w(p) (the empty-residual fallback) and the argmax of p (the empty-
//          row fallback);
//   pick   (sequences): the chunk holding the target from the chunk sums, then
//          an exact scan of that chunk alone.
// Greedy mode: the chunk argmaxes of every node, then one walk.
// Every result passes between launches through the workspace; no counters,
// nothing needs clearing.
//
// The commit then moves each accepted node's key and value from cache row
// ctx + node to ctx + depth, in increasing depth (a node's index is at least
// its depth, so no move reads a row an earlier move wrote).
#include "sv_common.h"

namespace sv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 16;                 // chunk entries per thread
constexpr int kChunk = kThreads * kPer;  // vocabulary chunk of one workgroup
constexpr int kVec = kPer / 4;           // float4 loads per thread and row over a chunk
constexpr float kTwo32 = 4294967296.0f;
typedef unsigned long long u64;

__device__ __forceinline__ u64 weight_of(float r) { return static_cast<u64>(fmaxf(r, 0.f) * kTwo32); }

// argmax combine: larger value wins, lower index on ties (order-independent)
__device__ __forceinline__ void amax(float &v, int &i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

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
// The residual after a second rejection, before its shift:
// max(0, R1 * SQ - Q * S1).
__device__ __forceinline__ U128 resid2_raw(u64 r1, u64 sq, float qe, u64 s1) {
  return subsat128(mul64(r1, sq), mul64(weight_of(qe), s1));
}

// ---- workspace ----------------------------------------------------------------

// Chunk results of one node: sums of w(p), w(p - q), w(q) and the argmax of p.
struct NodePart {
  u64 s0, s1, sq;
  float mv;
  int mi;
};
// How a sequence's walk ended.
enum DrawMode : int { kDone = 0, kDrawP = 1, kDrawR1 = 2, kDrawR2 = 3, kNeedSums = 4 };
struct DrawDesc {
  int row;    // stacked row of the node the token is drawn at (kNeedSums: the walk's node)
  int mode;   // DrawMode
  int p1;     // first residual replaced by w(p) (its sum was 0)
  int depth;  // the walk's depth at that node
  u64 s1, sq;  // first residual's sum (after that replacement) and sum Q
};
// Chunk results of a draw row: sum of the draw weights, of w(p), argmax of p.
struct DrawPart {
  u64 sres, sp;
  float mv;
  int mi;
  u64 pad;
};

struct TreeWs {
  u64 *rbuf;       // [B][V] residual of a node finished by its walk workgroup alone
  NodePart *np;    // [T][nchunk]
  int *need;       // [T] node whose chunk sums the second walk pass may use
  DrawDesc *desc;  // [B]
  U128 *p2;        // [B][nchunk] unshifted second-residual chunk sums
  DrawPart *p3;    // [B][nchunk]
  int nchunk;
  int vec;  // rows start 16-byte aligned and V % 4 == 0: float4 loads
};

constexpr size_t kWsAlign = 256;
inline size_t ws_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }
inline int chunks_of(int V) { return (V + kChunk - 1) / kChunk; }

// Region offsets of the workspace (each 256-byte aligned); returns the total.
constexpr int kRegions = 6;
size_t carve_offsets(int B, int V, long long T, size_t off[kRegions]) {
  const size_t nc = static_cast<size_t>(chunks_of(V));
  const size_t sz[kRegions] = {(size_t)B * V * sizeof(u64),      (size_t)T * nc * sizeof(NodePart),
                               (size_t)T * sizeof(int),          (size_t)B * sizeof(DrawDesc),
                               (size_t)B * nc * sizeof(U128),    (size_t)B * nc * sizeof(DrawPart)};
  size_t o = 0;
  for (int k = 0; k < kRegions; ++k) {
    off[k] = o;
    o = ws_up(o + sz[k]);
  }
  return o;
}

TreeWs carve(unsigned char *base, int B, int V, long long T) {
  size_t off[kRegions];
  carve_offsets(B, V, T, off);
  TreeWs w{};
  w.rbuf = reinterpret_cast<u64 *>(base + off[0]);
  w.np = reinterpret_cast<NodePart *>(base + off[1]);
  w.need = reinterpret_cast<int *>(base + off[2]);
  w.desc = reinterpret_cast<DrawDesc *>(base + off[3]);
  w.p2 = reinterpret_cast<U128 *>(base + off[4]);
  w.p3 = reinterpret_cast<DrawPart *>(base + off[5]);
  w.nchunk = chunks_of(V);
  return w;
}

// ---- block-wide reductions over the 256 threads -----------------------------

struct RedShared {
  u64 a[kWaves], b[kWaves], c[kWaves];
  float v[kWaves];
  int i[kWaves];
};

// Sums of three u64 values and an argmax; every thread gets the result.
__device__ void block_reduce(u64 &a, u64 &b, u64 &c, float &v, int &ix, RedShared &sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
    c += __shfl_xor(c, o);
    const float v2 = __shfl_xor(v, o);
    const int i2 = __shfl_xor(ix, o);
    amax(v, ix, v2, i2);
  }
  if (lane == 0) {
    sh.a[w] = a;
    sh.b[w] = b;
    sh.c[w] = c;
    sh.v[w] = v;
    sh.i[w] = ix;
  }
  __syncthreads();
  a = b = c = 0;
  v = -INFINITY;
  ix = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    a += sh.a[k];
    b += sh.b[k];
    c += sh.c[k];
    amax(v, ix, sh.v[k], sh.i[k]);
  }
  __syncthreads();
}

// 128-bit sum; every thread gets the result.
__device__ U128 block_add128(U128 x, RedShared &sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const U128 y{__shfl_xor(x.hi, o), __shfl_xor(x.lo, o)};
    x = add128(x, y);
  }
  if (lane == 0) {
    sh.a[w] = x.hi;
    sh.b[w] = x.lo;
  }
  __syncthreads();
  U128 t{0ull, 0ull};
#pragma unroll
  for (int k = 0; k < kWaves; ++k) t = add128(t, U128{sh.a[k], sh.b[k]});
  __syncthreads();
  return t;
}

// Exclusive prefix sum in thread order; *total gets the sum.
__device__ u64 block_exscan(u64 v, u64 *total, RedShared &sh) {
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
  for (int k = 0; k < kWaves; ++k) {
    if (k < w) before += sh.a[k];
    tot += sh.a[k];
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

// Probabilities of one row as the rule reads them: the entries themselves,
// or (logits rows) formed from the logits and the row's (max, sum) exactly as
// the head's softmax finish forms them.
struct PX {
  bool on;
  float Mk, S;
  __device__ __forceinline__ float operator()(float v) const { return on ? prob_of_logit(v, Mk, S) : v; }
};
__device__ __forceinline__ PX px_of(const TreeAcceptParams &p, int row) {
  if (!p.row_ms) return PX{false, 0.f, 1.f};
  return PX{true, p.row_ms[2 * row] * kLog2eF, p.row_ms[2 * row + 1]};
}

// Calls f(x, p(x), q(x)) on this thread's share of [x0, x1), x0 a chunk start
// (q(x) = 0 without q; p(x) through xf).  vec: all of the thread's float4
// loads first.
template <class F>
__device__ __forceinline__ void chunk_for(const float *pr, const float *qr, int x0, int x1, bool vec, const PX &xf,
                                          F &&f) {
  if (vec) {
    const float4 *p4 = reinterpret_cast<const float4 *>(pr);
    const float4 *q4 = reinterpret_cast<const float4 *>(qr);
    float4 pv[kVec], qv[kVec];
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
      const int x = x0 / 4 + threadIdx.x + k * kThreads;
      const bool in = x < x1 / 4;
      pv[k] = in ? p4[x] : make_float4(0.f, 0.f, 0.f, 0.f);
      qv[k] = (qr && in) ? q4[x] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
      const int x = x0 / 4 + threadIdx.x + k * kThreads;
      if (x >= x1 / 4) continue;
      f(4 * x, xf(pv[k].x), qv[k].x);
      f(4 * x + 1, xf(pv[k].y), qv[k].y);
      f(4 * x + 2, xf(pv[k].z), qv[k].z);
      f(4 * x + 3, xf(pv[k].w), qv[k].w);
    }
  } else {
    for (int x = x0 + threadIdx.x; x < x1; x += kThreads) f(x, xf(pr[x]), qr ? qr[x] : 0.f);
  }
}

// Sequence owning stacked row r: the largest i with q_start[i] <= r.
__device__ __forceinline__ int seq_of(const TreeAcceptParams &p, int r) {
  int lo = 0, hi = p.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.q_start[mid] <= r)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// ---- sums: chunk results of the nodes the walk needs them for -----------------

__global__ __launch_bounds__(kThreads) void tree_sums_kernel(TreeAcceptParams p, TreeWs w) {
  __shared__ RedShared sh;
  const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int V = p.V, x0 = c * kChunk, x1 = min(V, x0 + kChunk);
  const float *pr = p.p + (size_t)r * V;
  u64 s0 = 0, s1 = 0, sq = 0;
  float mv = -INFINITY;
  int mi = 0x7fffffff;
  if (p.greedy) {
    chunk_for(pr, nullptr, x0, x1, w.vec != 0, px_of(p, r), [&](int x, float pe, float) { amax(mv, mi, pe, x); });
  } else {
    if (!w.need[r]) return;  // flagged by the first walk pass
    chunk_for(pr, p.q + (size_t)r * V, x0, x1, w.vec != 0, px_of(p, r), [&](int, float pe, float qe) {
      s0 += weight_of(pe);
      s1 += weight_of(pe - qe);
      sq += weight_of(qe);
    });
  }
  block_reduce(s0, s1, sq, mv, mi, sh);
  if (tid == 0) w.np[(size_t)r * w.nchunk + c] = NodePart{s0, s1, sq, mv, mi};
}

// ---- walk ----------------------------------------------------------------------

struct WalkShared {
  int par[kMaxTreeNodes];
  int tok[kMaxTreeNodes];
  int path[kMaxTreeNodes];
  int first_kid[kMaxTreeNodes];
  int next_sib[kMaxTreeNodes];
  int nkids[kMaxTreeNodes];
  u64 anc[kMaxTreeNodes];  // bit m: node m is the node or one of its ancestors
  // each node's own test inputs: its uniform, and p and q of its parent's row at its token
  float ua[kMaxTreeNodes], pd[kMaxTreeNodes], qd[kMaxTreeNodes];
  int bad;
  int step, arg;
  int ok, result;
  u64 red64[kThreads];
  U128 red128[kThreads];
  float amax_v[kThreads];
  int amax_i[kThreads];
};

// Tree-based reductions of the workgroup-alone path (order fixed by the
// thread layout; integer sums do not depend on it anyway).
__device__ u64 walk_sum64(u64 v, WalkShared &sh) {
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

__device__ U128 walk_sum128(U128 v, WalkShared &sh) {
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
__device__ int walk_argmax(const float *row, const PX &xf, int V, WalkShared &sh) {
  const int tid = threadIdx.x;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int x = tid; x < V; x += kThreads) amax(bv, bi, xf(row[x]), x);
  sh.amax_v[tid] = bv;
  sh.amax_i[tid] = bi;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
      float v = sh.amax_v[tid];
      int ix = sh.amax_i[tid];
      amax(v, ix, sh.amax_v[tid + s], sh.amax_i[tid + s]);
      sh.amax_v[tid] = v;
      sh.amax_i[tid] = ix;
    }
    __syncthreads();
  }
  const int r = sh.amax_i[0] == 0x7FFFFFFF ? 0 : sh.amax_i[0];
  __syncthreads();
  return r;
}

// The least x whose running sum of R exceeds t (t < sum R): each thread owns
// one contiguous segment; segment sums are scanned in thread order.
__device__ int walk_draw(const u64 *R, int V, u64 t, WalkShared &sh) {
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

// Node v finished by the workgroup alone, the residual in R[V]: returns the
// child that passed, or -1 with *y the drawn token.
__device__ int walk_node_alone(const TreeAcceptParams &p, WalkShared &sh, int i, int qs, int n, int v,
                               u64 *R, int *y) {
  const int tid = threadIdx.x, V = p.V;
  const float *pv = p.p + (size_t)(qs + v) * V;
  const PX xf = px_of(p, qs + v);
  const float *qv = p.q + (size_t)(qs + v) * V;
  bool have_r = false;  // R holds the residual of the rejected children
  u64 S = 0, SQ = 0;
  bool sq_ready = false;
  for (int c = sh.first_kid[v]; c >= 0; c = sh.next_sib[c]) {
    const int d = sh.tok[c];
    if (!have_r) {
      if (tid == 0) sh.ok = (p.u_acc[qs + c] * qv[d] < xf(pv[d])) ? 1 : 0;
    } else {
      if (!sq_ready) {
        u64 part = 0;
        for (int x = tid; x < V; x += kThreads) part += weight_of(qv[x]);
        SQ = walk_sum64(part, sh);
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
    if (ok) return c;
    // rejected: the residual becomes the target
    if (!have_r) {
      u64 part = 0;
      for (int x = tid; x < V; x += kThreads) {
        const u64 wx = weight_of(xf(pv[x]) - qv[x]);
        R[x] = wx;
        part += wx;
      }
      S = walk_sum64(part, sh);
      have_r = true;
    } else {
      U128 part{0ull, 0ull};
      for (int x = tid; x < V; x += kThreads) part = add128(part, resid2_raw(R[x], SQ, qv[x], S));
      const U128 tot = walk_sum128(part, sh);
      const int shift = max(0, bitlen128(tot) - 32);
      // every thread rewrites only the entries it read
      u64 part2 = 0;
      for (int x = tid; x < V; x += kThreads) {
        const u64 wx = shr128_lo(resid2_raw(R[x], SQ, qv[x], S), shift);
        R[x] = wx;
        part2 += wx;
      }
      S = walk_sum64(part2, sh);
    }
    if (S == 0) {  // empty residual: back to the target row
      u64 part = 0;
      for (int x = tid; x < V; x += kThreads) {
        const u64 wx = weight_of(xf(pv[x]));
        R[x] = wx;
        part += wx;
      }
      S = walk_sum64(part, sh);
    }
  }
  // no child passed: draw from the residual (a node reaches here only after
  // rejections, so R is set)
  __syncthreads();  // R complete before the segment scan reads it
  if (S == 0) {
    *y = walk_argmax(pv, xf, V, sh);
  } else {
    u64 t = static_cast<u64>(floor(static_cast<double>(p.u_samp[i]) * static_cast<double>(S)));
    if (t > S - 1) t = S - 1;
    *y = walk_draw(R, V, t, sh);
  }
  return -1;
}

enum Step : int { kMove = 0, kEnd = 1, kDraw = 2, kAlone = 3, kNeed = 4 };

// The walk of one tree, one workgroup.  pass 0: greedy (chunk argmaxes of
// every node ready).  pass 1: stochastic, no chunk sums yet; a node whose
// first child is rejected and which has a second stops the walk, flagging
// that node and the nodes with two or more children below the second child
// (the only ones the walk can go on to without a third test).  pass 2: the
// walks that stopped go on with those nodes' sums; any other node that needs
// sums is finished by the workgroup alone.
__global__ __launch_bounds__(kThreads) void tree_walk_kernel(TreeAcceptParams p, TreeWs w, int pass) {
  __shared__ WalkShared sh;
  const int i = blockIdx.x, tid = threadIdx.x;
  const int qs = p.q_start[i], n = p.q_start[i + 1] - qs;
  const int V = p.V, nc = w.nchunk;
  int v = 0, depth = 0;
  if (pass == 2) {
    const DrawDesc dd = w.desc[i];
    if (dd.mode != kNeedSums) return;
    v = dd.row - qs;
    depth = dd.depth;
  }
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
  if (sh.bad) {  // (a second pass never sees a bad tree: the first left it done)
    if (tid == 0) {
      set_err(p.err, sh.bad);
      p.accepted[i] = -1;
      p.next_token[i] = -1;
      w.desc[i] = DrawDesc{qs, kDone, 0, 0, 0ull, 0ull};
      for (int k = 0; k < kMaxTreeNodes; ++k) p.path[(size_t)i * kMaxTreeNodes + k] = -1;
    }
    if (pass == 1)
      for (int j = tid; j < n; j += kThreads) w.need[qs + j] = 0;
    return;
  }
  // children in index order, child counts, ancestor sets, and every node's
  // own test inputs (gathered once: the walk then reads only LDS)
  for (int j = tid; j < n; j += kThreads) {
    int fk = -1, ns = -1, nk = 0;
    for (int c = n - 1; c > j; --c)
      if (sh.par[c] == j) {
        fk = c;
        ++nk;
      }
    if (j > 0)
      for (int c = j + 1; c < n; ++c)
        if (sh.par[c] == sh.par[j]) {
          ns = c;
          break;
        }
    u64 m = 1ull;
    for (int x = j; x > 0; x = sh.par[x]) m |= 1ull << x;
    sh.first_kid[j] = fk;
    sh.next_sib[j] = ns;
    sh.nkids[j] = nk;
    sh.anc[j] = m;
    if (!p.greedy && j > 0) {
      const size_t at = (size_t)(qs + sh.par[j]) * V + sh.tok[j];
      sh.ua[j] = p.u_acc[qs + j];
      sh.pd[j] = px_of(p, qs + sh.par[j])(p.p[at]);
      sh.qd[j] = p.q[at];
    }
  }
  if (pass == 2) {
    for (int k = tid; k <= depth; k += kThreads) sh.path[k] = p.path[(size_t)i * kMaxTreeNodes + k];
  } else if (tid == 0) {
    sh.path[0] = 0;
  }
  __syncthreads();

  int y = -1;
  bool drawn_here = false;
  for (;;) {
    // one step of the walk, decided by thread 0 from LDS and chunk totals
    if (tid == 0) {
      const NodePart *np = w.np + (size_t)(qs + v) * nc;
      int step = kEnd, arg = 0;
      if (p.greedy) {
        float mv = -INFINITY;
        int mi = 0x7fffffff;
        for (int cc = 0; cc < nc; ++cc) amax(mv, mi, np[cc].mv, np[cc].mi);
        if (mi == 0x7fffffff) mi = 0;
        int c = sh.first_kid[v];
        while (c >= 0 && sh.tok[c] != mi) c = sh.next_sib[c];
        step = c >= 0 ? kMove : kEnd;
        arg = c >= 0 ? c : mi;
      } else {
        DrawDesc dd{qs + v, kDrawP, 0, depth, 0ull, 0ull};
        const int c1 = sh.first_kid[v];
        step = kDraw;  // a leaf: the bonus token from p_v
        if (c1 >= 0) {
          const int c2 = sh.next_sib[c1];
          if (sh.ua[c1] * sh.qd[c1] < sh.pd[c1]) {
            step = kMove;
            arg = c1;
          } else if (c2 < 0) {
            dd.mode = kDrawR1;  // the only child rejected
          } else if (pass == 1) {
            step = kNeed;
            arg = c2;
            dd.mode = kNeedSums;
          } else if (!w.need[qs + v]) {
            step = kAlone;
          } else {
            u64 S0 = 0, S1 = 0, SQ = 0;
            for (int cc = 0; cc < nc; ++cc) {
              S0 += np[cc].s0;
              S1 += np[cc].s1;
              SQ += np[cc].sq;
            }
            const int p1 = S1 == 0;  // empty first residual: w(p) instead
            if (p1) S1 = S0;
            const u64 U = static_cast<u64>(static_cast<double>(sh.ua[c2]) * 16777216.0);
            const u64 R1 = p1 ? weight_of(sh.pd[c2]) : weight_of(sh.pd[c2] - sh.qd[c2]);
            if (less128(mul64(U * weight_of(sh.qd[c2]), S1), shl128(mul64(R1, SQ), 24))) {
              step = kMove;
              arg = c2;
            } else if (sh.next_sib[c2] < 0) {
              dd = DrawDesc{qs + v, kDrawR2, p1, depth, S1, SQ};  // both children rejected
            } else {
              step = kAlone;  // a third sibling's test needs the second residual's sum
            }
          }
        }
        if (step == kDraw || step == kNeed) w.desc[i] = dd;
      }
      sh.step = step;
      sh.arg = arg;
    }
    __syncthreads();
    const int step = sh.step, arg = sh.arg;
    __syncthreads();
    if (step == kMove) {
      v = arg;
      ++depth;
      if (tid == 0) sh.path[depth] = v;
      continue;
    }
    if (step == kEnd) {
      y = arg;
      drawn_here = true;
      break;
    }
    if (step == kNeed) {
      // sums for v and for the nodes of two or more children below its
      // second child; the path so far, for the second pass
      for (int j = tid; j < n; j += kThreads)
        w.need[qs + j] = (j == v || (((sh.anc[j] >> arg) & 1ull) && sh.nkids[j] >= 2)) ? 1 : 0;
      for (int k = tid; k <= depth; k += kThreads) p.path[(size_t)i * kMaxTreeNodes + k] = sh.path[k];
      return;
    }
    if (step == kDraw) break;
    const int c = walk_node_alone(p, sh, i, qs, n, v, w.rbuf + (size_t)i * V, &y);
    if (c >= 0) {
      v = c;
      ++depth;
      if (tid == 0) sh.path[depth] = v;
      continue;
    }
    drawn_here = true;
    break;
  }
  if (pass == 1)
    for (int j = tid; j < n; j += kThreads) w.need[qs + j] = 0;
  __syncthreads();
  if (tid == 0) {
    p.accepted[i] = depth;
    p.kv_len[i] += depth + 1;
    if (drawn_here) {
      p.next_token[i] = y;
      w.desc[i] = DrawDesc{qs + v, kDone, 0, depth, 0ull, 0ull};
    }
  }
  for (int k = tid; k < kMaxTreeNodes; k += kThreads)
    p.path[(size_t)i * kMaxTreeNodes + k] = k <= depth ? sh.path[k] : -1;
}

// ---- the draw ------------------------------------------------------------------

// Shift of the second residual: the bit length of its total beyond 32.
__device__ int resid2_shift(const TreeWs &w, int i, RedShared &sh) {
  U128 t{0ull, 0ull};
  for (int cc = threadIdx.x; cc < w.nchunk; cc += kThreads) t = add128(t, w.p2[(size_t)i * w.nchunk + cc]);
  return max(0, bitlen128(block_add128(t, sh)) - 32);
}

// The draw's weight of one entry (ur = 0: the fallback w(p)).
struct DrawWeight {
  int mode, p1, ur, shift;
  u64 s1, sq;
  __device__ __forceinline__ u64 operator()(float pe, float qe) const {
    if (!ur || mode == kDrawP) return weight_of(pe);
    const u64 r1 = p1 ? weight_of(pe) : weight_of(pe - qe);
    if (mode == kDrawR1) return r1;
    return shr128_lo(resid2_raw(r1, sq, qe, s1), shift);
  }
};

__global__ __launch_bounds__(kThreads) void tree_resid2_kernel(TreeAcceptParams p, TreeWs w) {
  __shared__ RedShared sh;
  const int c = blockIdx.x, i = blockIdx.y;
  const DrawDesc dd = w.desc[i];
  if (dd.mode != kDrawR2) return;
  const int V = p.V, x0 = c * kChunk, x1 = min(V, x0 + kChunk);
  U128 acc{0ull, 0ull};
  chunk_for(p.p + (size_t)dd.row * V, p.q + (size_t)dd.row * V, x0, x1, w.vec != 0, px_of(p, dd.row),
            [&](int, float pe, float qe) {
              const u64 r1 = dd.p1 ? weight_of(pe) : weight_of(pe - qe);
              acc = add128(acc, resid2_raw(r1, dd.sq, qe, dd.s1));
            });
  acc = block_add128(acc, sh);
  if (threadIdx.x == 0) w.p2[(size_t)i * w.nchunk + c] = acc;
}

__global__ __launch_bounds__(kThreads) void tree_draw_sums_kernel(TreeAcceptParams p, TreeWs w) {
  __shared__ RedShared sh;
  const int c = blockIdx.x, i = blockIdx.y;
  const DrawDesc dd = w.desc[i];
  if (dd.mode == kDone) return;
  const int V = p.V, x0 = c * kChunk, x1 = min(V, x0 + kChunk);
  const DrawWeight f{dd.mode, dd.p1, 1, dd.mode == kDrawR2 ? resid2_shift(w, i, sh) : 0, dd.s1, dd.sq};
  u64 sres = 0, sp = 0, z = 0;
  float mv = -INFINITY;
  int mi = 0x7fffffff;
  const float *qr = dd.mode == kDrawP ? nullptr : p.q + (size_t)dd.row * V;
  chunk_for(p.p + (size_t)dd.row * V, qr, x0, x1, w.vec != 0, px_of(p, dd.row), [&](int x, float pe, float qe) {
    sres += f(pe, qe);
    sp += weight_of(pe);
    amax(mv, mi, pe, x);
  });
  block_reduce(sres, sp, z, mv, mi, sh);
  if (threadIdx.x == 0) w.p3[(size_t)i * w.nchunk + c] = DrawPart{sres, sp, mv, mi, 0ull};
}

__global__ __launch_bounds__(kThreads) void tree_pick_kernel(TreeAcceptParams p, TreeWs w) {
  __shared__ RedShared sh;
  __shared__ int s_found, s_hit, s_res;
  __shared__ u64 s_target;
  const int i = blockIdx.x, tid = threadIdx.x;
  const DrawDesc dd = w.desc[i];
  if (dd.mode == kDone) return;
  const int V = p.V, nc = w.nchunk;
  const DrawPart *pp = w.p3 + (size_t)i * nc;
  u64 sres = 0, sp = 0, z = 0;
  float mv = -INFINITY;
  int mi = 0x7fffffff;
  for (int cc = tid; cc < nc; cc += kThreads) {
    sres += pp[cc].sres;
    sp += pp[cc].sp;
    amax(mv, mi, pp[cc].mv, pp[cc].mi);
  }
  block_reduce(sres, sp, z, mv, mi, sh);
  // weights: the draw's own, else w(p) (empty residual), else the argmax
  const int ur = sres > 0 ? 1 : (sp > 0 ? 0 : -1);
  int result = mi == 0x7fffffff ? 0 : mi;
  if (ur >= 0) {
    const int shift = (ur && dd.mode == kDrawR2) ? resid2_shift(w, i, sh) : 0;
    const DrawWeight f{dd.mode, dd.p1, ur, shift, dd.s1, dd.sq};
    const u64 S = ur ? sres : sp;
    u64 t = static_cast<u64>(floor(static_cast<double>(p.u_samp[i]) * static_cast<double>(S)));
    if (t >= S) t = S - 1;
    // the chunk holding t: chunk sums scanned in order, 256 at a time
    if (tid == 0) {
      s_found = 0;
      s_hit = nc - 1;
      s_target = 0;
    }
    __syncthreads();
    u64 run = 0;
    for (int base = 0; base < nc; base += kThreads) {
      const int cc = base + tid;
      const u64 v = cc < nc ? (ur ? pp[cc].sres : pp[cc].sp) : 0ull;
      u64 tot;
      const u64 before = run + block_exscan(v, &tot, sh);
      if (v > 0 && before <= t && t < before + v) {
        s_found = 1;
        s_hit = cc;
        s_target = t - before;
      }
      run += tot;
      __syncthreads();
      if (s_found) break;
    }
    // exact scan of that chunk: each thread a contiguous segment
    const int cx0 = s_hit * kChunk, cn = min(V, cx0 + kChunk) - cx0;
    const float *pr = p.p + (size_t)dd.row * V + cx0;
    const PX xf = px_of(p, dd.row);
    const float *qr = (ur && dd.mode != kDrawP) ? p.q + (size_t)dd.row * V + cx0 : nullptr;
    const bool vec = w.vec != 0;
    int per = (cn + kThreads - 1) / kThreads;  // <= kPer
    if (vec) per = (per + 3) & ~3;             // whole float4s (cn % 4 == 0 here)
    const int lo = min(cn, tid * per), hi = min(cn, lo + per);
    u64 wv[kPer];
    u64 s = 0;
    if (vec) {
      const float4 *p4 = reinterpret_cast<const float4 *>(pr + lo);
      const float4 *q4 = reinterpret_cast<const float4 *>(qr ? qr + lo : pr);
      const int n4 = (hi - lo) / 4;
      float4 pv[kVec], qv[kVec];
#pragma unroll
      for (int k = 0; k < kVec; ++k) {
        pv[k] = k < n4 ? p4[k] : make_float4(0.f, 0.f, 0.f, 0.f);
        qv[k] = (qr && k < n4) ? q4[k] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < kVec; ++k) {
        const bool in = k < n4;
        wv[4 * k] = in ? f(xf(pv[k].x), qv[k].x) : 0ull;
        wv[4 * k + 1] = in ? f(xf(pv[k].y), qv[k].y) : 0ull;
        wv[4 * k + 2] = in ? f(xf(pv[k].z), qv[k].z) : 0ull;
        wv[4 * k + 3] = in ? f(xf(pv[k].w), qv[k].w) : 0ull;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int x = lo + k;
        wv[k] = x < hi ? f(xf(pr[x]), qr ? qr[x] : 0.f) : 0ull;
      }
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) s += wv[k];
    u64 tot;
    const u64 before = block_exscan(s, &tot, sh);
    const u64 tt = s_target;
    if (tid == 0) s_res = cx0 + cn - 1;  // (t lies in this chunk)
    __syncthreads();
    if (s > 0 && before <= tt && tt < before + s) {
      u64 acc = before;
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        acc += wv[k];
        if (acc > tt) {
          s_res = cx0 + lo + k;
          break;
        }
      }
    }
    __syncthreads();
    result = s_res;
  }
  if (tid == 0) p.next_token[i] = result;
}

// Row moves of the commit, one workgroup per (sequence, KV head); T is the
// cache element (bf16 bits, or int8 codes whose per-vector scales move too).
template <class T>
__device__ __forceinline__ void commit_rows(const TreeCommitParams &p, int i, int h) {
  const int tid = threadIdx.x;
  const int a = p.accepted[i];
  if (a <= 0) return;
  const int ctx = p.kv_len[i] - a - 1;
  const int *path = p.path + (size_t)i * kMaxTreeNodes;
  T *kc = static_cast<T *>(p.kc[i]) + (size_t)h * p.kv_cap * p.hd;
  T *vc = static_cast<T *>(p.vc[i]) + (size_t)h * p.hd * p.kv_cap;
  float *ks = p.kv8 ? static_cast<float *>(p.ksc[i]) + (size_t)h * p.kv_cap : nullptr;
  float *vs = p.kv8 ? static_cast<float *>(p.vsc[i]) + (size_t)h * p.kv_cap : nullptr;
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
      if (ks && tid == 0) {
        ks[dst] = ks[src];
        vs[dst] = vs[src];
      }
    }
    __syncthreads();  // depth k lands before depth k + 1 reads
  }
}

__global__ __launch_bounds__(kThreads) void tree_commit_kernel(TreeCommitParams p) {
  if (p.kv8)
    commit_rows<int8_t>(p, blockIdx.x, blockIdx.y);
  else
    commit_rows<uint16_t>(p, blockIdx.x, blockIdx.y);
}

}  // namespace

size_t tree_workspace_bytes(int B, int V, long long T) {
  size_t off[kRegions];
  return carve_offsets(B, V, T, off);
}

hipError_t launch_tree_accept(const TreeAcceptParams &p, hipStream_t s) {
  const long long T = p.q_start[p.B];
  TreeWs w = carve(p.ws, p.B, p.V, T);
  const uintptr_t al = reinterpret_cast<uintptr_t>(p.p) | reinterpret_cast<uintptr_t>(p.greedy ? p.p : p.q);
  w.vec = (p.V % 4) == 0 && (al % 16) == 0;
  const dim3 blk(kThreads);
  trace_before(SV_K_ACCEPT, s);
  const dim3 all_rows(w.nchunk, static_cast<unsigned>(T));
  if (p.greedy) {
    hipLaunchKernelGGL(tree_sums_kernel, all_rows, blk, 0, s, p, w);
    hipLaunchKernelGGL(tree_walk_kernel, dim3(p.B), blk, 0, s, p, w, 0);
  } else {
    hipLaunchKernelGGL(tree_walk_kernel, dim3(p.B), blk, 0, s, p, w, 1);
    hipLaunchKernelGGL(tree_sums_kernel, all_rows, blk, 0, s, p, w);
    hipLaunchKernelGGL(tree_walk_kernel, dim3(p.B), blk, 0, s, p, w, 2);
    hipLaunchKernelGGL(tree_resid2_kernel, dim3(w.nchunk, p.B), blk, 0, s, p, w);
    hipLaunchKernelGGL(tree_draw_sums_kernel, dim3(w.nchunk, p.B), blk, 0, s, p, w);
    hipLaunchKernelGGL(tree_pick_kernel, dim3(p.B), blk, 0, s, p, w);
  }
  trace_after(SV_K_ACCEPT, s);
  return hipGetLastError();
}

hipError_t launch_tree_commit(const TreeCommitParams &p, hipStream_t s) {
  hipLaunchKernelGGL(tree_commit_kernel, dim3(p.B, p.hkv), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace sv
