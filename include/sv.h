/*
 * sv.h -- batched speculative verification on AMD Instinct MI355X (gfx950).
 *
 * B sequences each carry gamma_i drafted tokens.  One target-model pass
 * verifies all sum(gamma_i + 1) stacked tokens with a single read of the
 * weights, rejection sampling keeps each sequence's accepted prefix plus one
 * token of the target's own, and only the KV lengths are committed: no
 * sequence is padded to the longest run.
 *
 * Source passages (pages of the method's write-ups):
 *  - "Speculative Decoding and Batching Compete for the Same Compute Slack on
 *    RDNA4": FAQ on the ragged tensor problem and section "The batch also goes
 *    ragged" (per-sequence positions, masks and KV lengths; padding or
 *    realignment are the costs to avoid); sections "The budget is fixed, and
 *    the batch is inside it" and "What the budget says to build" (draft
 *    length as a function of the live batch).
 *  - "Speculative Decoding at High Batch Size: Where the 3x Speedup Turns
 *    Into a Tax": sections "What does one speculative iteration actually
 *    cost?" and "How does the roofline model work?" (expected tokens, step
 *    model, crossover batch); rejection sampling keeps the output distribution
 *    of plain decoding (section "Why do the headline speedups all come from
 *    batch 1?").
 *  - the speculative-decoding primer (splicedso.github.io/learn), section
 *    "The idea": one pass checks every draft, keeps the drafts up to the first
 *    rejection and adds one token of its own.
 *
 * Conventions for every call:
 *  - Pointers are device pointers owned by the caller unless marked (host).
 *    The library keeps no pointer after a call returns and never allocates or
 *    frees device memory inside these calls; scratch memory comes from a
 *    caller workspace sized by the matching *_workspace_bytes query.
 *  - Work is enqueued on the caller's HIP stream (`stream` is a hipStream_t;
 *    NULL is the null stream).  No call synchronises the stream or the device;
 *    outputs are valid once the stream reaches that point.
 *  - The return value is an sv_status.  Arguments are validated on the host
 *    before anything is enqueued; a failing call enqueues nothing, except
 *    SV_ERR_HIP, which reports a failed launch (hipGetLastError is consumed).
 *  - Errors that depend on device data (a token id outside the vocabulary, a
 *    KV length that would overflow the cache) set bits in the optional device
 *    word *err_flag (SV_DEV_ERR_*) and never write outside caller buffers.
 *  - Workspaces: zero-fill a workspace once after allocating it.  Its first
 *    256 KiB hold the library's arrival counters in every call; each call
 *    leaves them zeroed again, so one workspace (sized for the largest call)
 *    can serve later calls of any kind on the same stream.  Calls that overlap
 *    in time must use different workspaces.
 *  - Thread safety: calls may come from several host threads; the only
 *    global state is the optional kernel-timing trace (sv_trace_*) and the
 *    launch-policy override (sv_set_gemm_tuning).
 */
#ifndef SV_H
#define SV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sv_status;

#define SV_OK 0
#define SV_ERR_INVALID_ARG (-1) /* null pointer, negative size, inconsistent counts */
#define SV_ERR_UNSUPPORTED (-2) /* a shape or dtype the library does not handle */
#define SV_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required */
#define SV_ERR_HIP (-4)         /* a kernel launch failed */
#define SV_ERR_TOO_LARGE (-5)   /* the call needs more scratch than the fixed array of
                                   sv_accept_commit_noalloc holds */

/* Device-side error bits, OR-ed into *err_flag. */
#define SV_DEV_ERR_BAD_TOKEN 1   /* token id outside [0, vocab) */
#define SV_DEV_ERR_KV_OVERFLOW 2 /* kv_len[i] + gamma_i + 1 > kv_cap */
#define SV_DEV_ERR_BAD_TREE 8    /* a tree node whose parent is not an earlier node */
#define SV_DEV_ERR_CTX_BOUND 4   /* kv_len[i] > max_ctx: that sequence gets no attention
                                    work and its output rows are unspecified; the other
                                    sequences' results are unaffected */

/* Layer kinds (sv_layer.kind). */
#define SV_LAYER_EMBED 0   /* x[t] = E[token[t]] */
#define SV_LAYER_DECODER 1 /* one pre-norm decoder layer */
#define SV_LAYER_HEAD 2    /* final RMSNorm, LM head, softmax */

/* Weight storage (sv_layer.wtype). */
#define SV_W_F32 0      /* fp32 [N][K] */
#define SV_W_BF16 1     /* bf16 [N][K] */
#define SV_W_INT4_G32 2 /* int4, groups of 32 along K: packed uint32 [N][K/8],
                           nibble i of word m = code + 8 for k = 8m + i,
                           codes in [-7, 7]; bf16 scales [N][K/32];
                           weight = code * scale */

/* Weight layouts (sv_layer.layout). */
#define SV_LAYOUT_ROWMAJOR 0 /* [N][K] as described below */
#define SV_LAYOUT_PACKED 1   /* produced by sv_pack_matrix (bf16 and int4 only) */

/* sv_verify_layer flags. */
#define SV_HEAD_LOGITS 1       /* HEAD: write fp32 logits instead of probabilities */
#define SV_HEAD_LOGITS_STATS 2 /* HEAD: write fp32 logits [T][vocab] followed by each
                                  row's (max, sum of exp(logit - max)) [T][2]; feeds
                                  sv_accept_commit with SV_ACCEPT_FROM_LOGITS */

/* One weight matrix in [N][K] = [output features][reduction] layout.
 * scale is used only for SV_W_INT4_G32. */
typedef struct sv_matrix {
  const void *w;
  const void *scale;
} sv_matrix;

/* Layer description (host struct).
 *
 * DECODER computes, for the stacked verify tokens x[T][d] (bf16):
 *   h = RMSNorm(x) (eps, unit gain);  q, k, v = h Wq^T, h Wk^T, h Wv^T;
 *   RoPE on q and k at each token's position, pairs (i, i + head_dim/2)
 *   rotated by pos * rope_theta^(-2i/head_dim);
 *   k and v appended to the sequence's cache at that position (bf16);
 *   o = softmax(q K^T / sqrt(head_dim)) V, query j of sequence i seeing keys
 *   0 .. kv_len[i] + j, query head h reading KV head h / (n_q_heads/n_kv_heads);
 *   x1 = x + o Wo^T;  y = x1 + (silu(RMSNorm(x1) Wg^T) * (RMSNorm(x1) Wu^T)) Wd^T.
 * HEAD computes logits = RMSNorm(y) Wlm^T and p = softmax(logits) per row.
 * EMBED copies E[token] (fp32 or bf16 table [vocab][d]) to bf16 rows.
 *
 * Shapes: Wq [n_q*hd][d], Wk/Wv [n_kv*hd][d], Wo [d][n_q*hd], Wg/Wu [ffn][d],
 * Wd [d][ffn], lm_head [vocab][d], embed [vocab][d].
 * Supported: d, ffn, n_q*hd multiples of 64; head_dim 64 or 128;
 * n_q_heads a multiple of n_kv_heads. */
typedef struct sv_layer {
  int32_t kind;
  int32_t wtype;
  int32_t layout;     /* SV_LAYOUT_*, for every GEMM matrix of the layer */
  int32_t d;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn;
  int32_t vocab;
  float eps;          /* RMSNorm epsilon (1e-6 in the reference model) */
  float rope_theta;   /* RoPE base (1e4 in the reference model) */
  sv_matrix wq, wk, wv, wo, w_gate, w_up, w_down; /* DECODER */
  sv_matrix embed;    /* EMBED: table, wtype SV_W_F32 or SV_W_BF16 */
  sv_matrix lm_head;  /* HEAD */
} sv_layer;

/* Batch description (host struct; the arrays it points to are as marked).
 *
 * Token map: sequence i owns stacked rows q_start[i] .. q_start[i] + gamma_i
 * where q_start is the exclusive prefix sum of (gamma_i + 1); row j of
 * sequence i is the token at position kv_len[i] + j (j = 0 is the last
 * committed token, j >= 1 the drafts).  T must equal sum(gamma_i + 1).
 *
 * KV caches: k_cache[i] points to sequence i's keys, bf16 [n_kv][kv_cap][hd]
 * (position-major); v_cache[i] to its values, bf16 in blocks of 32
 * positions, [n_kv][kv_cap/32][hd][32] (value (head h, position p, column c)
 * at ((h * kv_cap/32 + p/32) * hd + c) * 32 + p % 32: one head's values for
 * 32 consecutive positions form one contiguous [hd][32] block).  Entries at
 * positions < kv_len[i] are read; the pass writes positions kv_len[i] ..
 * kv_len[i] + gamma_i.  kv_cap is a multiple of 32; every cache base is
 * 16-byte aligned (the kernels read and write them with 8- and 16-byte
 * accesses). */
typedef struct sv_batch {
  int32_t B;                 /* sequences, >= 0 */
  int32_t T;                 /* stacked tokens = sum(gamma_i + 1) */
  int32_t max_ctx;           /* upper bound on every kv_len[i] (sizes the attention grid;
                                a sequence with a larger kv_len is skipped by attention
                                and sets SV_DEV_ERR_CTX_BOUND) */
  int32_t kv_cap;            /* cache capacity per sequence, multiple of 32 */
  const int32_t *gamma_host; /* (host) [B] draft counts, >= 0 */
  const int32_t *gamma;      /* [B] the same counts on the device */
  const int32_t *kv_len;     /* [B] cached tokens before the pass */
  void *const *k_cache;      /* [B] device pointers */
  void *const *v_cache;      /* [B] device pointers */
  int32_t *err_flag;         /* [1] nullable */
  /* Token trees (NULL for the linear pass): sequence i's stacked rows are
   * then the nodes 0 .. gamma_i of a tree in topological order (node 0 the
   * last committed token, gamma_i + 1 <= 64), and tree_parent[q_start[i] + j]
   * is node j's parent (< j; ignored for node 0).  Node j is at position
   * kv_len[i] + depth(j) (its rotary angle), its key and value are appended
   * at cache row kv_len[i] + j, and it attends to keys 0 .. kv_len[i] - 1 and
   * to the rows of its ancestors and itself.  A parent that is not an earlier
   * node sets SV_DEV_ERR_BAD_TREE (that node's outputs are unspecified). */
  const int32_t *tree_parent; /* [T] */
  /* KV cache storage: SV_KV_BF16 (the layouts above) or SV_KV_INT8: the same
   * layouts with one int8 code per value, and per sequence the fp32 scales of
   * every cached vector, k_scale[i] / v_scale[i] -> [n_kv][kv_cap] (value =
   * code * scale).  The pass stores its new keys and values the same way:
   * rounded to bf16, then scale = absmax / 127 over the head's vector (fp32,
   * correctly rounded), code = clamp(rne(x / scale), -127, 127) (0 for an
   * all-zero vector).  The query-row limit per KV head (GQA group x
   * (gamma_i + 1) <= 128) is the same as for bf16 caches. */
  int32_t kv_dtype;
  void *const *k_scale; /* [B] device pointers (SV_KV_INT8) */
  void *const *v_scale; /* [B] */
} sv_batch;

#define SV_KV_BF16 0
#define SV_KV_INT8 1

/* Packed weight layout.  Rows are taken in 32-row groups g (G = ceil(N/32)
 * groups), each made of two 16-row tiles a = 0, 1, stored step-major: for K
 * step s, group 0's fragments, then group 1's, ..., then step s + 1.  A GEMM
 * unit of 32 rows reads one contiguous run per K step, and units working on
 * the same step read neighbouring memory:
 *   bf16: for step s (k = 64s..64s+63), group g, tile a, half m, lane l
 *         (row 32g + 16a + l%16), the 8 values k = 64s + 32m + 8(l/16) + 0..7
 *         are stored at element (((s * G + g) * 2 + a) * 2 + m) * 512 + l * 8;
 *   int4: for step s (k = 128s..128s+127), group g, tile a, lane l, the 32
 *         codes k = 128s + 32(l/16) + 0..31 of row 32g + 16a + l%16 (four
 *         packed words) are stored at word (((s * G + g) * 2 + a) * 64 + l) * 4,
 *         and their group scale at element ((s * G + g) * 2 + a) * 64 + l of
 *         the scale array.
 * Rows past N in the last group are zero.  Packing is a one-time layout
 * change (done when weights are loaded), not part of a verification pass. */
sv_status sv_packed_matrix_bytes(int32_t wtype, int32_t N, int32_t K, size_t *w_bytes,
                                 size_t *scale_bytes);

/* Pack a row-major [N][K] matrix (and its int4 scales) into the packed
 * layout on `stream`.  Destinations must not overlap the sources. */
sv_status sv_pack_matrix(int32_t wtype, int32_t N, int32_t K, const void *w, const void *scale,
                         void *w_packed, void *scale_packed, void *stream);

/* Workspace needed by sv_verify_layer for this layer, batch and flags. */
sv_status sv_verify_layer_workspace_bytes(const sv_layer *layer, const sv_batch *batch,
                                          int32_t flags, size_t *bytes);

/* One verify pass through one layer.
 *
 * Defined by: "Speculative Decoding at High Batch Size: Where the 3x Speedup
 * Turns Into a Tax", section "Why do the headline speedups all come from
 * batch 1?" (one target pass checks every drafted token of every sequence
 * with a single read of the weights), and "Speculative Decoding and Batching
 * Compete for the Same Compute Slack on RDNA4", section "The batch also goes
 * ragged" and its FAQ on the ragged tensor problem (each sequence keeps its
 * own draft count, positions, causal mask and KV length; no padding).
 *
 *   DECODER: x_in bf16 [T][d] -> y_out bf16 [T][d]; appends K/V rows.
 *   HEAD:    x_in bf16 [T][d] -> y_out fp32 [T][vocab] probabilities
 *            (or logits with SV_HEAD_LOGITS; or logits followed by the rows'
 *            softmax statistics, T * (vocab + 2) floats, with
 *            SV_HEAD_LOGITS_STATS).
 *   EMBED:   x_in int32 token ids [T] -> y_out bf16 [T][d].
 * x_in and y_out must not overlap.  Only B, T, gamma_host and err_flag of the
 * batch are used by EMBED and HEAD. */
sv_status sv_verify_layer(const sv_layer *layer, const sv_batch *batch, const void *x_in,
                          void *y_out, int32_t flags, void *workspace, size_t workspace_bytes,
                          void *stream);

/* Acceptance modes, optionally or'ed with SV_ACCEPT_FROM_LOGITS: p is then
 * the output of an SV_HEAD_LOGITS_STATS head call (logits [T][V] followed by
 * each row's (max M, sum S of exp(logit - M)) [T][2]) and every probability
 * the rule reads is formed from it exactly as the head's softmax finish
 * forms it (exp2(logit * log2 e - M log2 e) / S in fp32), so the results are
 * bit-identical to passing the head's probabilities. */
#define SV_ACCEPT_STOCHASTIC 0
#define SV_ACCEPT_GREEDY 1
#define SV_ACCEPT_FROM_LOGITS 0x100

/* Workspace needed by sv_accept_commit. */
sv_status sv_accept_commit_workspace_bytes(int32_t B, int32_t V, int32_t mode,
                                           const int32_t *gamma_host, size_t *bytes);

/* Acceptance, resampling and commit for every sequence (rejection sampling
 * in the sense of Leviathan, Kalman and Matias).
 *
 * Defined by: the speculative-decoding primer (splicedso.github.io/learn),
 * section "The idea" (keep the drafts up to the first rejection, then one
 * token of the target's own: 3 of 4 accepted gives 4 tokens, none gives 1);
 * "Speculative Decoding at High Batch Size: Where the 3x Speedup Turns Into
 * a Tax", section "Why do the headline speedups all come from batch 1?" (the
 * rejection-sampling rule keeps the target's output distribution); and
 * "Speculative Decoding and Batching Compete for the Same Compute Slack on
 * RDNA4", section "The batch also goes ragged" (sequences accept different
 * lengths; only each sequence's KV length is committed, nothing realigned).
 *
 * Rows: p row q_start[i] + j (j = 0..gamma_i) is the target distribution of
 * the (j+1)-th new token of sequence i; q row q_start[i] - i + j
 * (j = 0..gamma_i - 1) is the draft distribution of draft token j+1, whose id
 * is draft[q_start[i] - i + j].  p fp32 [T][V], q fp32 [sum gamma][V], with
 * entries in [0, 1].  u_acc fp32 [sum gamma], u_samp fp32 [B] in [0, 1).
 *
 * Stochastic mode, per sequence:
 *   a = number of leading drafts with fl32(u_acc * q(d)) < p(d);
 *   r = max(0, fl32(p_{a+1} - q_{a+1})) if a < gamma_i, else p_{gamma_i+1};
 *   R(x) = trunc(fl32(r(x) * 2^32)) as 64-bit integers, S = sum R (exact);
 *   if S == 0 after a rejection, R is taken from p_{a+1}; if S is still 0
 *   the token is argmax p_{a+1} (lowest index);
 *   t = floor(fl64(u_samp * S)) (at most S - 1); next_token = least x whose
 *   running sum of R exceeds t.
 * Greedy mode: a = leading drafts equal to argmax p_j, next_token =
 * argmax p_{a+1} (lowest index on ties); q, u_acc, u_samp may be NULL.
 * Commit: accepted[i] = a, kv_len[i] += a + 1 (in place).  A sequence whose
 * drafts contain an id outside [0, V) is left uncommitted: accepted and
 * next_token are -1, kv_len unchanged, SV_DEV_ERR_BAD_TOKEN set. */
sv_status sv_accept_commit(int32_t B, int32_t V, int32_t mode, const int32_t *gamma_host,
                           const int32_t *gamma, const int32_t *draft, const float *p,
                           const float *q, const float *u_acc, const float *u_samp,
                           int32_t *kv_len, int32_t *accepted, int32_t *next_token,
                           int32_t *err_flag, void *workspace, size_t workspace_bytes,
                           void *stream);

/* sv_accept_commit without a workspace, for callers that cannot allocate
 * device memory or hand the library a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Arguments
 * and results are those of sv_accept_commit (bit-identical outputs).  The
 * scratch memory comes from a fixed device array of
 * SV_ACCEPT_NOALLOC_SCRATCH_BYTES that each GPU holds from the library's first
 * call on it until the process ends; the call allocates and frees nothing.
 * Every call on one GPU shares that array, so calls that overlap in time on
 * one GPU (other streams, other threads) race: serialise them.  A call whose
 * scratch would exceed the array (about B * 4 + rows * ceil(V / chunk) * 24 +
 * (B + T) * 4 bytes, rows = B stochastic or T greedy, chunk 4096 or 8192)
 * returns SV_ERR_TOO_LARGE before enqueueing anything. */
#define SV_ACCEPT_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
sv_status sv_accept_commit_noalloc(int32_t B, int32_t V, int32_t mode, const int32_t *gamma_host,
                                   const int32_t *gamma, const int32_t *draft, const float *p,
                                   const float *q, const float *u_acc, const float *u_samp,
                                   int32_t *kv_len, int32_t *accepted, int32_t *next_token,
                                   int32_t *err_flag, void *stream);

/* Token-tree acceptance and commit.
 *
 * Defined by: "Speculative Decoding and Batching Compete for the Same Compute
 * Slack on RDNA4", section "What the budget says to build" (Table 1: a lone
 * agent spends its slack on "a small tree, ~8 to 16 deep" of candidates) and
 * the page's opening (the tree rides under the weight stream of one verify
 * pass); the acceptance keeps the target's distribution as the rejection
 * rule of sv_accept_commit does ("Speculative Decoding at High Batch Size:
 * Where the 3x Speedup Turns Into a Tax", section "Why do the headline
 * speedups all come from batch 1?").
 *
 * Sequence i's stacked rows q_start[i] .. q_start[i] + gamma_i are the nodes
 * of a tree in topological order (node 0 = the last committed token);
 * parent[t] is the node's parent within its tree (< its own index; ignored
 * for node 0), tokens[t] its token.  p fp32 [T][V]: target row of each node
 * (the distribution of the token after it, e.g. an SV_LAYER_HEAD output over
 * a tree verify pass); q fp32 [T][V]: the draft distribution each node's
 * children were drawn from (independently); u_acc [T]: one uniform per node
 * for its own test (node 0's unused); u_samp [B].  Uniforms in [0, 1) on the
 * 2^-24 grid.
 * Stochastic mode walks down from the root; at node v the children are tested
 * in index order: the first passes iff fl32(u * q_v(d)) < p_v(d); after a
 * rejection the target is the integer residual R (first
 * trunc(fl32(max(0, fl32(p_v - q_v)) * 2^32)), sum S) and a later child d
 * passes iff U * Q(d) * S < R(d) * SQ * 2^24 (U = u * 2^24,
 * Q = trunc(fl32(q_v * 2^32)), SQ = sum Q); each further rejection sets
 * R = max(0, R * SQ - Q * S) shifted right until its sum fits 32 bits.  The
 * first passing child becomes v; with none, or at a leaf, next_token is drawn
 * from R (or from trunc(fl32(p_v * 2^32)), the bonus row) by the inverse-CDF
 * rule of sv_accept_commit.  On a chain (one child per node) this is exactly
 * sv_accept_commit.  Greedy mode follows the child whose token is argmax p_v
 * (lowest index on ties); q, u_acc, u_samp may be NULL.  Either mode may be
 * or'ed with SV_ACCEPT_FROM_LOGITS: p is then the output of an
 * SV_HEAD_LOGITS_STATS head call over the tree pass, and every probability
 * is formed from it as sv_accept_commit forms it (bit-identical results).
 * Outputs: accepted[i] = depth of the last accepted node, next_token[i],
 * kv_len[i] += accepted[i] + 1, path (device int32 [B][64]): the accepted node
 * at each depth (path[i][0] = 0), -1 past the end.  A tree with a bad parent
 * (SV_DEV_ERR_BAD_TREE) or token (SV_DEV_ERR_BAD_TOKEN) is left uncommitted
 * (accepted = next_token = -1).  B <= 256, gamma_i + 1 <= 64 nodes. */
sv_status sv_accept_tree_workspace_bytes(int32_t B, int32_t V, const int32_t *gamma_host,
                                         size_t *bytes);
sv_status sv_accept_tree(int32_t B, int32_t V, int32_t mode, const int32_t *gamma_host,
                         const int32_t *parent, const int32_t *tokens, const float *p,
                         const float *q, const float *u_acc, const float *u_samp,
                         int32_t *kv_len, int32_t *accepted, int32_t *next_token, int32_t *path,
                         int32_t *err_flag, void *workspace, size_t workspace_bytes, void *stream);

/* The tree commit's cache-row moves for one layer's caches (call once per
 * layer after sv_accept_tree): the accepted node at depth k moves from row
 * ctx + path[i][k] to ctx + k, ctx = kv_len[i] - accepted[i] - 1 (kv_len and
 * accepted as sv_accept_tree left them).  Caches as in sv_batch (K
 * [n_kv][kv_cap][head_dim], V in 32-position blocks); sequences with
 * accepted <= 0 are untouched. */
sv_status sv_tree_commit_kv(int32_t B, int32_t n_kv_heads, int32_t head_dim, int32_t kv_cap,
                            const int32_t *kv_len, const int32_t *accepted, const int32_t *path,
                            void *const *k_cache, void *const *v_cache, void *stream);

/* The same moves for int8 caches (sv_batch with SV_KV_INT8: codes in the
 * bf16 layouts, one byte per value; k_scale / v_scale: per sequence, fp32
 * [n_kv][kv_cap], one scale per cached vector): each moved vector's codes
 * and scale.  Defined by the same passages as sv_tree_commit_kv, with the
 * caches of "Why Static Batching Wastes an RX 9070 XT Agent Swarm and
 * Continuous Batching Wins It Back", section "The catch is prefill, and it
 * points back at admission" (quantised KV). */
sv_status sv_tree_commit_kv_int8(int32_t B, int32_t n_kv_heads, int32_t head_dim, int32_t kv_cap,
                                 const int32_t *kv_len, const int32_t *accepted, const int32_t *path,
                                 void *const *k_cache, void *const *v_cache, void *const *k_scale,
                                 void *const *v_scale, void *stream);

/* Iteration-level batching (host only).
 *
 * Defined by: "Why Static Batching Wastes an RX 9070 XT Agent Swarm and
 * Continuous Batching Wins It Back", sections "What a draining batch actually
 * costs" (a static batch keeps finished lanes as padding until its longest
 * member stops; a shrinking one drops them) and "Continuous batching refills
 * the slot instead of freezing it" (membership decided every step, a
 * finished sequence's slot refilled from the queue on the next step).
 *
 * A scheduler of `slots` lanes serves submitted requests (each needing a
 * number of tokens) in submission order; request ids are 0, 1, 2, ...
 * Per step: sv_sched_next fills slot_request[slots] (request per lane, -1
 * empty) and live[slots] (1 where that request still needs tokens; static
 * batches keep finished lanes as padding, live 0) and *width (lanes the step
 * carries, padding included; 0 once nothing is left); the caller runs the
 * verify pass over the lanes and reports each lane's emitted tokens (for a
 * verify pass accepted + 1) with sv_sched_commit, which returns the useful
 * tokens of the step (emissions past a request's need are not counted).  A
 * handle is used by one thread at a time. */
#define SV_SCHED_STATIC 0
#define SV_SCHED_SHRINK 1
#define SV_SCHED_CONTINUOUS 2
typedef struct sv_sched sv_sched;
sv_status sv_sched_create(int32_t slots, int32_t policy, sv_sched **out);
sv_status sv_sched_destroy(sv_sched *sched);
sv_status sv_sched_submit(sv_sched *sched, int32_t tokens, int32_t *request_out);
sv_status sv_sched_next(sv_sched *sched, int32_t *slot_request, int32_t *live, int32_t *width);
sv_status sv_sched_commit(sv_sched *sched, const int32_t *emitted, int32_t *useful_out);

/* Per-position acceptance counters, accumulated over calls.
 *
 * Defined by: "Speculative Decoding at High Batch Size: Where the 3x Speedup
 * Turns Into a Tax", section "How do you measure this on your own server?"
 * (log acceptance per position and turn it into a conditional rate: position
 * k accepted given position k-1 was) -- the rates SV_PLAN_SPEEDUP takes as
 * its per-position acceptance.
 *
 * For the gamma[B] and accepted[B] of an sv_accept_commit call (device
 * arrays), adds to counts (device, int64 [2][n_pos], zero it before the first
 * call):  counts[0][k-1] += sequences that tested draft k (gamma_i >= k and
 * accepted_i >= k - 1),  counts[1][k-1] += sequences that accepted it
 * (accepted_i >= k), for k = 1..n_pos (1 <= n_pos <= 256).  Sequences left
 * uncommitted (accepted_i < 0) are skipped.  counts[1][k] / counts[0][k] is
 * the conditional acceptance rate at position k + 1.  Integer adds: the
 * totals do not depend on the order of the additions. */
sv_status sv_accept_position_counts(int32_t B, int32_t n_pos, const int32_t *gamma,
                                    const int32_t *accepted, int64_t *counts, void *stream);

/* Draft-length planning (host only). */
#define SV_PLAN_BUDGET 0  /* keep sum(gamma_i + 1) within the compute-slack budget */
#define SV_PLAN_SPEEDUP 1 /* maximise the step-model speedup over plain decoding */

typedef struct sv_plan_params {
  int32_t mode;
  int32_t gamma_max;       /* cap on any gamma_i */
  int32_t budget_tokens;   /* BUDGET: slack in tokens; 0 = floor(t_floor_ms / c_ms) */
  int32_t fill_remainder;  /* BUDGET: give the leftover tokens to the first sequences */
  double t_floor_ms;       /* decode step floor (BUDGET when budget_tokens == 0) */
  double t_w_ms;           /* weight-read time per step */
  double k_ms;             /* KV-read time per sequence */
  double c_ms;             /* compute time per token */
  double draft_frac;       /* drafter size relative to the target (e.g. 0.04) */
  int32_t n_alpha;         /* 1: independent acceptance alpha[0]; >1: conditional
                              acceptance per position (last value repeats) */
  const double *alpha;     /* (host) [n_alpha] */
} sv_plan_params;

/* Draft lengths for the live batch.
 *
 * Defined by: BUDGET -- "Speculative Decoding and Batching Compete for the
 * Same Compute Slack on RDNA4", sections "The budget is fixed, and the batch
 * is inside it" and "What the budget says to build" (Table 1: the slack of
 * one decode step, in tokens, less one committed token per live sequence,
 * split over the sequences); SPEEDUP -- "Speculative Decoding at High Batch
 * Size: Where the 3x Speedup Turns Into a Tax", sections "What does one
 * speculative iteration actually cost?" (expected tokens and the speedup
 * ratio) and "How does the roofline model work?" (step time and the
 * crossover batch B*).
 *
 * gamma_out (host) [B_live] receives the draft lengths.
 * BUDGET: n = budget tokens; if B_live >= n every gamma is 0, otherwise the
 *   n - B_live free tokens are split evenly (floor), the first
 *   (n - B_live) mod B_live sequences getting one more if fill_remainder,
 *   each capped at gamma_max.
 * SPEEDUP: one gamma in 0..gamma_max for all sequences, maximising
 *   E(gamma) t(B,1) / (t(B, gamma+1) + t_d(B, gamma)) with
 *   t(B, n) = max(t_w + B k, B n c), t_d(B, g) = max(f t_w + B k, f B g c);
 *   ties go to the smaller gamma.
 * *bstar_out (nullable) receives the crossover batch t_w / ((g+1) c - k) for
 * the largest planned g (infinity when the denominator is <= 0 or t_w, c
 * are not given). */
sv_status sv_plan_gamma(const sv_plan_params *params, int32_t B_live, int32_t *gamma_out,
                        double *bstar_out);

/* Kernel-timing trace (profiling aid).  While a trace is active, every
 * stride-th launch of the named kernel class (the 1st, the (stride+1)-th, ...)
 * is bracketed by a pair of HIP events on the launch stream, up to `capacity`
 * bracketed launches (timing-only events, recorded without a system-scope
 * fence; each record still costs a few microseconds of stream time, which a
 * stride above 1 spreads thinner).  sv_trace_end synchronises the device,
 * writes the elapsed milliseconds of each bracketed launch to ms_out (host,
 * capacity entries), stores their number in *count and releases the events.
 * One trace at a time; SV_ERR_INVALID_ARG for a bad class, capacity or
 * stride, or while another trace is active. */
#define SV_K_GEMM_QKV 0
#define SV_K_ATTENTION 1
/* 2: unused (the attention kernel merges its chunks itself) */
#define SV_K_GEMM_O 3
#define SV_K_GEMM_GATE_UP 4
#define SV_K_GEMM_DOWN 5
#define SV_K_GEMM_LM_HEAD 6
#define SV_K_SOFTMAX 7
#define SV_K_ACCEPT 8
#define SV_K_PREP 9
#define SV_K_EMBED 10
#define SV_K_COUNT 11

sv_status sv_trace_begin(int32_t kernel_class, int32_t capacity, int32_t stride);
sv_status sv_trace_end(float *ms_out, int32_t capacity, int32_t *count);

/* Launch-policy override for the GEMMs of later sv_verify_layer calls (and
 * their workspace sizes), for tuning sweeps and tests; results stay within
 * the same error bounds, though the summation order changes.  spec is a
 * comma-separated list of kind:splits:depth[:waves] entries, kind one of
 * qkv, o, gu, down, head; splits = K splits across workgroups, depth = K steps
 * in flight per wave (2, 4 or 8), waves = waves of one workgroup sharing a
 * unit's K range (1, 4, 8 or 16), or for many stacked tokens 0 (the
 * LDS-tiled kernel), 2 (the wide streaming kernel) or 3 (the square-tiled
 * kernel), bf16 packed weights only (the wide kernel also needs more than 16
 * tokens; otherwise the policy's choice stays).  Zero splits or depth, or an absent kind, keep the default
 * policy; settings beyond a kernel's register budget fall back to the nearest
 * smaller one.  NULL restores the defaults (also read from the environment
 * variable SV_GEMM_TUNE when the library loads).  Process-wide; set it
 * between calls, not while another thread is inside the library.
 * SV_ERR_INVALID_ARG for a malformed spec (the setting is unchanged). */
sv_status sv_set_gemm_tuning(const char *spec);

/* Message for a status code (static string). */
const char *sv_status_string(sv_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t sv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SV_H */
