// Internal declarations shared by the gfx950 kernels and the host dispatch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sv.h"

namespace sv {

// ---------------------------------------------------------------------------
// Vector types for the CDNA4 matrix cores.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// D = A(16x32) * B(32x16) + C, bf16 inputs, fp32 accumulate.
// Lane l: A row l%16, k = 8*(l/16)..+7; B column l%16, same k; D rows
// 4*(l/16)..+3 of column l%16.
__device__ __forceinline__ floatx4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b,
                                                const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> a packed bf16 pair (a in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// fp32 -> bf16, round to nearest even.
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) {
  return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// Fragment layout of a bf16 activation matrix [T][K] (the token operand of the
// short-projection GEMMs): for each K step s of 64 and 16-token tile, two
// 1 KiB fragments m = 0, 1 in MFMA lane order, lane (gq, l16) holding the
// eight values x[16 tile + l16][64 s + 32 m + 8 gq ..]; ntt tiles per step.
// A wave then loads each fragment as one contiguous 1 KiB access instead of
// sixteen 64-byte row pieces.
__host__ __device__ inline size_t frag_index(int t, int k, int ntt) {
  const int s = k >> 6, m = (k >> 5) & 1, gq = (k >> 3) & 3, e = k & 7;
  return ((((size_t)s * ntt + (t >> 4)) * 2 + m) * 64 + gq * 16 + (t & 15)) * 8 + e;
}

// ---------------------------------------------------------------------------
// Block-level helpers (blockDim.x == 256).

// In-place exclusive prefix sum of n (<= 65536) ints in LDS; returns the total.
// tmp: 257 ints of LDS (the first 4 are used).  Each thread sums a contiguous
// segment; the segment sums are scanned with wave shuffles and the four wave
// totals added in wave order.  Deterministic (integer sums).
__device__ inline int block_exscan(int *vals, int n, int *tmp) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (n + 255) / 256;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += vals[i];
  int inc = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int v = tmp[k];
    if (k < w) before += v;
    total += v;
  }
  int run = before + inc - s;
  for (int i = lo; i < hi; ++i) {
    const int v = vals[i];
    vals[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

// Largest i in [0, n) with starts[i] <= x (starts ascending, starts[0] <= x).
__device__ inline int upper_index(const int *starts, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (starts[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline void set_err(int *err, int bits) {
  if (err) atomicOr(err, bits);
}

// ---------------------------------------------------------------------------
// Kernel parameter blocks.

constexpr int kMaxB = 65536;        // sequences per call (LDS token-map limit)
constexpr int kAttnMaxChunks = 32;  // attention work items (key chunks) per sequence
constexpr int kAttnMaxRows = 128;   // query rows per (sequence, KV head): GQA group x tokens
constexpr int kScanMaxB = 4096;     // kernels that keep the full map in LDS

enum RowMap { RM_LINEAR = 0, RM_ROPE_PAIRS = 1, RM_SWIGLU = 2 };
enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };
enum WType { WT_F32 = 0, WT_BF16 = 1, WT_INT4 = 2 };

struct GemmMat {
  const void *w;
  const uint16_t *s;
  int rows;
};

struct GemmParams {
  const uint16_t *x;  // activations bf16 [T][K]
  const uint16_t *xp; // the same in fragment layout (ntt = xp_ntt), or nullptr
  int xp_ntt;
  uint16_t *out_pk;   // EPI_RESID: also write the output in fragment layout;
  int out_pk_ntt;     // EPI_SWIGLU: write it only in fragment layout (nullptr: row-major)
  int T, K, N;        // N = logical rows
  int nmat;
  GemmMat mat[3];
  int rowmap, hd;
  int packed;          // weights in the packed fragment layout
  int splits, ksteps;  // ksteps = K / step size
  int nblk, ntblk;     // 32-row groups (16 features for SWIGLU), token blocks
  const float *rnorm;      // per-token RMSNorm scale [T] (nullptr: see rparts / none)
  const float *rparts;     // per-token sums of squares in nparts partials [T][nparts]
  int nparts;
  int rms_inline;          // one-wave-per-unit launches without K split: the RMSNorm
                           // scale from the token operand the workgroup loads
  float eps;
  float *sq_out;           // EPI_RESID: sums of squares of the output, [T][row groups]
  float *partial;      // K-split partial tiles (device-scope stores)
  int *counters;       // [ntblk * nblk] arrival counters, zero between launches
  int epi;
  void *out;
  int ldo;
  const uint16_t *resid;  // EPI_RESID
  float *stats;           // EPI_LOGITS: [T][nblk][2] (max, sum exp of the group)
  // EPI_QKV
  uint16_t *qbuf;  // [T][hq][hd]
  int hq, hkv;
  const int *tok_seq;  // [T] sequence of each stacked token
  const int *tok_pos;  // [T] its position
  const float *rope_cs;  // [T][hd/2][2] rotation cos, sin
  int B, kv_cap;
  void *const *kc;
  void *const *vc;
  uint16_t *kvstage;  // int8 caches: the new keys / values go here instead, [T][2][hkv][hd] bf16
  int *err;
};

struct PrepParams {
  const uint16_t *x;   // [T][d] rows whose RMSNorm scale is needed
  int T, d;
  float eps;
  float *rnorm;        // [T]
  // token map (decoder calls; gamma == nullptr skips it)
  const int *gamma;
  const int *kv_len;
  int B, chunk;
  int *tok_seq;        // [T]
  int *tok_pos;        // [T]
  int *q_start;        // [B + 1]
  int *chunk_start;    // [B + 1] attention work items of each sequence
  float *rope_cs;      // [T][hd/2][2] cos, sin (nullptr: none)
  int hd;
  const int *tree_parent;        // [T] token trees: parent of each node (nullptr: chains)
  unsigned long long *tree_mask; // [T] out: ancestor-or-self mask of each node
  int4 *items;         // [max_items][2] attention work items (see AttnParams)
  int max_items;
  int max_ctx;         // the host's bound on kv_len (a longer sequence is flagged, not attended)
  uint16_t *xp;        // x in fragment layout for the QKV GEMM (nullptr: none)
  int xp_ntt;
  int *err;
  double inv_freq[64]; // theta^(-2i/hd), i < hd/2 (evaluated on the host in fp64)
};

// Attention work item (written by the prep pass, two int4 per item):
//   [0] = {sequence (-1: no work), first key, end key, gamma}
//   [1] = {kv_len, first stacked row of the sequence, the sequence's first item,
//          its number of items}
struct AttnParams {
  const uint16_t *qbuf;  // [T][hq][hd] (rotated)
  const int4 *items;     // [max_items][2]
  const unsigned long long *tree_mask;  // [T] visible new keys per row (nullptr: causal chain)
  void *const *kc;
  void *const *vc;
  int B, T, hq, hkv, hd, kv_cap, max_ctx;
  int chunk;        // keys per work item
  int max_items;    // grid.x
  int rpad;         // padded query rows per (seq, kv head)
  float scale_log2; // log2(e) / sqrt(hd)
  float *part_o;    // [max_items][hkv][rpad][hd]
  float *part_ml;   // [max_items][hkv][rpad][2]
  uint16_t *out;    // [T][hq*hd], or in fragment layout when out_ntt > 0
  int out_ntt;
  int *counters;    // [B][hkv] arrival counters, zero between launches
  int *err;
  // int8 caches (kv8): codes in the bf16 layouts with one byte per value, and
  // per (head, position) fp32 scales [hkv][kv_cap] behind ksc[seq], vsc[seq]
  int kv8;
  void *const *ksc;
  void *const *vsc;
};

// Quantisation of the pass's new keys and values into int8 caches.
struct KvQuantParams {
  const uint16_t *kvstage;  // [T][2][hkv][hd] bf16
  const int *tok_seq, *tok_pos;
  int T, hkv, hd, kv_cap;
  void *const *kc;
  void *const *vc;
  void *const *ksc;
  void *const *vsc;
};
hipError_t launch_kv_quant(const KvQuantParams &p, hipStream_t s);

struct HeadSoftmaxParams {
  float *logits;        // [T][V] in: logits, out: probabilities
  const float *stats;   // [T][nblk][2]
  int T, V, nblk, cols_per_block;
  float *row_ms;        // row statistics kernel: [T][2] (max, sum of exp)
};

struct EmbedParams {
  const int *tokens;
  const void *table;  // [V][d] fp32 or bf16
  int table_bf16;
  int T, V, d;
  uint16_t *out;
  int *err;
};

struct AcceptPart {
  unsigned long long sum_res;  // residual / bonus weights in this chunk
  unsigned long long sum_p;    // fallback weights (target row)
  float max_p;                 // argmax of the target row in this chunk
  int arg_p;
};

constexpr int kAcceptHostMax = 256;  // batches up to this size get the token map with the launch

struct AcceptParams {
  int B, V, T, nd, mode;
  int chunk, nchunk;
  const int *gamma;
  const int *draft;
  const float *p;
  const float *row_ms;  // non-null: p holds logits, row_ms[row] = (max, sum of exp)
  const float *q;
  const float *u_acc;
  const float *u_samp;
  int *kv_len;
  int *accepted;
  int *next_token;
  int *err;
  AcceptPart *parts;   // stochastic: [B][nchunk]; greedy: [T][nchunk]
  int *acc_ws;         // [B + T] ints of spill space (greedy rows past the LDS table)
  int *counters;       // [B] arrival counters, zero between calls
  // small batches: the token map from the host's draft counts, passed with the
  // launch (no device pass over gamma before the first load)
  int host_map;                        // 1 when the two arrays below are filled
  int hq_start[kAcceptHostMax];        // q_start[i]
  int hgamma[kAcceptHostMax];          // gamma_i
};

// ---------------------------------------------------------------------------
// Host launchers (one per kernel family).  Return hipSuccess or the launch error.
// depth = K steps in flight per wave (2, 4, 8); kw = waves per unit (1, 4, 8, 16),
// kGemmTiled for the LDS-tiled kernel (bf16, packed weights, no K split), or
// kGemmWide for the wide streaming kernel (bf16, packed weights, tok_tiles 4
// or 8 per token block).
constexpr int kGemmTiled = -1;
constexpr int kGemmWide = -2;
constexpr int kGemmSquare = -3;  // 256 x 256 square-tiled kernel (bf16 packed, no K split)
hipError_t launch_gemm(const GemmParams &p, int wtype, int tok_tiles, int depth, int kw, hipStream_t s,
                       int trace_class);
hipError_t launch_pack(int wtype, int N, int K, const void *w, const void *scale, void *wp,
                       void *sp, hipStream_t s);
// Packed int4 [N][K] (+ scales) -> packed bf16, the values the int4 GEMM uses.
// Workspace floats for the K-split partial tiles of one GEMM launch.
size_t gemm_partial_floats(int ngroups, int splits, int ntblk, int tok_tiles);
hipError_t launch_prep(const PrepParams &p, hipStream_t s);
// rnorm[t] = 1 / sqrt(sum of parts[t][0 .. nparts) / K + eps)
hipError_t launch_rnorm_parts(const float *parts, int nparts, int T, int K, float eps, float *rnorm,
                              hipStream_t s);
hipError_t launch_attention(const AttnParams &p, hipStream_t s);
hipError_t launch_head_softmax(const HeadSoftmaxParams &p, hipStream_t s);
hipError_t launch_head_rowstats(const HeadSoftmaxParams &p, hipStream_t s);

// Probability of a logit from its row's (max M, sum S), exactly as the head's
// softmax finish computes it.
constexpr float kLog2eF = 1.4426950408889634f;
__device__ __forceinline__ float prob_of_logit(float l, float Mk, float S) {
  return __builtin_amdgcn_exp2f(fmaf(l, kLog2eF, -Mk)) / S;
}
hipError_t launch_embed(const EmbedParams &p, hipStream_t s);
hipError_t launch_accept(const AcceptParams &p, hipStream_t s);
constexpr int kMaxCountPositions = 256;  // positions a counter call can record

// Token trees: nodes per tree (ancestor masks are 64-bit) and sequences per
// tree-acceptance call (their row offsets travel with the launch).
constexpr int kMaxTreeNodes = 64;
constexpr int kTreeMaxB = 256;

struct TreeAcceptParams {
  int B, V, greedy;
  const int *parent;      // [T] parent node of each stacked node (roots: any)
  const int *tokens;      // [T] token of each node (roots: ignored)
  const float *p;         // [T][V] target rows: probabilities, or logits when row_ms is set
  const float *row_ms;    // [T][2] (max, sum of exp(logit - max)) of each logits row, or null
  const float *q;         // [T][V] draft distribution of each node's children
  const float *u_acc;     // [T] one uniform per node (its own test)
  const float *u_samp;    // [B]
  int *kv_len, *accepted, *next_token;
  int *path;              // [B][kMaxTreeNodes] accepted node at each depth, -1 past the end
  int *err;
  unsigned char *ws;      // workspace, tree_workspace_bytes(B, V, T) bytes
  int q_start[kTreeMaxB + 1];
};

// Workspace of one tree acceptance call over B sequences, T stacked nodes.
size_t tree_workspace_bytes(int B, int V, long long T);

struct TreeCommitParams {
  int B, hkv, hd, kv_cap;
  const int *kv_len, *accepted, *path;
  void *const *kc;
  void *const *vc;
  int kv8;              // int8 caches: one byte per value, and the scales below
  void *const *ksc;     // [B] fp32 [hkv][kv_cap] scale of each cached key (int8 caches)
  void *const *vsc;     // [B] the same for the values
};

hipError_t launch_tree_accept(const TreeAcceptParams &p, hipStream_t s);
hipError_t launch_tree_commit(const TreeCommitParams &p, hipStream_t s);
hipError_t launch_position_counts(int B, int n_pos, const int *gamma, const int *accepted,
                                  unsigned long long *counts, hipStream_t s);

// Acceptance call geometry and its scratch layout: arrival counters first
// (counter_bytes of room), then the per-chunk results and the spill space.
struct AcceptPlan {
  long long T = 0, nd = 0;
  int nchunk = 0, chunk = 0;
  size_t off_parts = 0, off_acc = 0, bytes = 0;
};
sv_status plan_accept(int32_t B, int32_t V, int32_t mode, const int32_t *gamma_host, AcceptPlan &ap,
                      size_t counter_bytes);
sv_status check_accept_args(int32_t B, int32_t mode, const AcceptPlan &ap, const int32_t *gamma,
                            const int32_t *draft, const float *p, const float *q, const float *u_acc,
                            const float *u_samp, const int32_t *kv_len, const int32_t *accepted,
                            const int32_t *next_token);
sv_status run_accept(int32_t B, int32_t V, int32_t mode, const int32_t *gamma_host, const AcceptPlan &ap,
                     const int32_t *gamma, const int32_t *draft, const float *p, const float *q,
                     const float *u_acc, const float *u_samp, int32_t *kv_len, int32_t *accepted,
                     int32_t *next_token, int32_t *err_flag, unsigned char *ws, hipStream_t stream);

// Kernel-timing trace hooks (host).
void trace_before(int kernel_class, hipStream_t s);
void trace_after(int kernel_class, hipStream_t s);

// Register budget of the GEMM instantiations: which (weight type, token
// tiles, waves per unit) combinations compile without spilling at 8 steps in
// flight (deep) and at 4.  Larger workgroups leave fewer registers per wave.
constexpr bool gemm_deep_ok(int wt, int tt, int kw) {
  return wt == WT_BF16 ? (kw <= 4 || (kw == 8 && tt <= 2)) : wt == WT_INT4 ? (tt <= 2 && kw <= 4) : false;
}
constexpr bool gemm_kw_ok(int wt, int tt, int kw) {
  return wt == WT_BF16   ? (kw <= 8 || tt <= 2)
         : wt == WT_INT4 ? (kw <= 4 || (kw == 8 && tt <= 2) || (kw == 16 && tt == 1))
                         : kw <= 8;
}

// Largest number of partial sums of squares per token (the previous
// projection's row groups) that a gate||up launch with several waves per unit
// stages in LDS (four-aligned counts, up to two token tiles); other gate||up
// launches take the scales from a separate reduction pass.
constexpr int kRsPartsMax = 160;
inline bool rs_parts_in_gemm(int kw, int tt, int nparts) {
  return kw > 1 && tt <= 2 && nparts > 0 && nparts % 4 == 0 && nparts <= kRsPartsMax;
}

// Step sizes along K per weight type.
inline int kstep_of(int wtype) { return wtype == WT_INT4 ? 128 : 64; }

}  // namespace sv
