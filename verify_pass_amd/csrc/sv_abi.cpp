// C-ABI entry points: argument validation, workspace layout, launch geometry
// and kernel dispatch on the caller's stream.  No allocation, no sync.
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "sv_common.h"

using namespace sv;

// ---------------------------------------------------------------------------
// Kernel-timing trace.
namespace {
struct TraceState {
  std::mutex mu;
  std::atomic<int> cls{-1};
  int cap = 0;
  int n = 0;
  int stride = 1;
  long long seen = 0;  // launches of the class since the trace began
  bool open = false;
  std::vector<hipEvent_t> ev;
};
TraceState g_trace;
}  // namespace

void sv::trace_before(int kernel_class, hipStream_t s) {
  if (g_trace.cls.load(std::memory_order_relaxed) != kernel_class) return;
  std::lock_guard<std::mutex> lk(g_trace.mu);
  const bool take = g_trace.seen++ % g_trace.stride == 0;
  if (take && g_trace.n < g_trace.cap && !g_trace.open) {
    if (hipEventRecord(g_trace.ev[2 * g_trace.n], s) == hipSuccess) g_trace.open = true;
  }
}

void sv::trace_after(int kernel_class, hipStream_t s) {
  if (g_trace.cls.load(std::memory_order_relaxed) != kernel_class) return;
  std::lock_guard<std::mutex> lk(g_trace.mu);
  if (g_trace.open) {
    (void)hipEventRecord(g_trace.ev[2 * g_trace.n + 1], s);
    g_trace.open = false;
    ++g_trace.n;
  }
}

extern "C" sv_status sv_trace_begin(int32_t kernel_class, int32_t capacity, int32_t stride) {
  if (kernel_class < 0 || kernel_class >= SV_K_COUNT || capacity <= 0 || stride <= 0) return SV_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_trace.mu);
  if (g_trace.cls.load() >= 0) return SV_ERR_INVALID_ARG;  // one trace at a time
  g_trace.ev.assign(2 * (size_t)capacity, nullptr);
  // timing-only events: no system-scope fence (cache write-back) at each record,
  // which would otherwise add a gap around every bracketed launch
  for (auto &e : g_trace.ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return SV_ERR_HIP;
  g_trace.cap = capacity;
  g_trace.stride = stride;
  g_trace.seen = 0;
  g_trace.n = 0;
  g_trace.open = false;
  g_trace.cls.store(kernel_class);
  return SV_OK;
}

extern "C" sv_status sv_trace_end(float *ms_out, int32_t capacity, int32_t *count) {
  std::lock_guard<std::mutex> lk(g_trace.mu);
  if (g_trace.cls.load() < 0) return SV_ERR_INVALID_ARG;
  g_trace.cls.store(-1);
  sv_status st = SV_OK;
  const int n = g_trace.n;
  if (n > 0 && (hipEventSynchronize(g_trace.ev[2 * n - 1]) != hipSuccess || hipDeviceSynchronize() != hipSuccess))
    st = SV_ERR_HIP;
  for (int i = 0; i < n && st == SV_OK; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_trace.ev[2 * i], g_trace.ev[2 * i + 1]) != hipSuccess) st = SV_ERR_HIP;
    if (ms_out && i < capacity) ms_out[i] = ms;
  }
  for (auto &e : g_trace.ev) (void)hipEventDestroy(e);
  g_trace.ev.clear();
  if (count) *count = n;
  g_trace.n = 0;
  g_trace.cap = 0;
  return st;
}

extern "C" const char *sv_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SV_ERR_WORKSPACE: return "workspace missing or too small";
    case SV_ERR_HIP: return "HIP launch failure";
    case SV_ERR_TOO_LARGE: return "the call needs more scratch than the fixed no-allocation array holds";
    default: return "unknown status";
  }
}

extern "C" int32_t sv_version(void) { return 100; }

// ---------------------------------------------------------------------------
// Planning of one verify_layer call.
namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
// Every workspace starts with the same fixed block of arrival counters, so a
// workspace zero-filled once stays valid when it is shared between calls of
// different kinds and shapes (each launch leaves the counters it used at 0).
constexpr size_t kCounterBytes = 256 * 1024;
constexpr int kSoftmaxCols = 8192;  // columns per softmax-finish workgroup (256 threads x 8 float4)
constexpr size_t kMaxCounters = kCounterBytes / sizeof(int);

// GEMM kinds of one pass (for the launch policy and its tuning override).
enum GemmKind { GK_QKV = 0, GK_O, GK_GU, GK_DOWN, GK_HEAD, GK_COUNT };

// Optional override of the launch policy (tuning sweeps, tests):
// "qkv:1:4:16,o:1:4:16,gu:1:8:4,down:1:8:16,head:1:2:1"
// (kind:splits:depth[:waves per unit, 0 = the LDS-tiled kernel, 2 = the wide
// streaming kernel, 3 = the square-tiled kernel]), from
// SV_GEMM_TUNE at load time or sv_set_gemm_tuning.
struct Tune {
  int splits[GK_COUNT];
  int depth[GK_COUNT];
  int kw[GK_COUNT];
};

bool parse_tune(const char *e, Tune &r) {
  for (int i = 0; i < GK_COUNT; ++i) {
    r.splits[i] = r.depth[i] = 0;
    r.kw[i] = -1;  // not set
  }
  if (!e) return true;
  const char *names[GK_COUNT] = {"qkv", "o", "gu", "down", "head"};
  for (int i = 0; i < GK_COUNT; ++i) {
    const char *f = std::strstr(e, names[i]);
    while (f && !((f == e || f[-1] == ',') && f[std::strlen(names[i])] == ':'))
      f = std::strstr(f + 1, names[i]);
    if (!f) continue;
    int s = 0, d = 0, k = 0;
    const int n = std::sscanf(f + std::strlen(names[i]), ":%d:%d:%d", &s, &d, &k);
    if (n < 2 || s < 0 || d < 0 || k < 0) return false;
    r.splits[i] = s;
    r.depth[i] = d;
    if (n == 3) r.kw[i] = k;
  }
  return true;
}

std::mutex g_tune_mu;
Tune g_tune = [] {
  Tune r;
  if (!parse_tune(std::getenv("SV_GEMM_TUNE"), r)) parse_tune(nullptr, r);
  return r;
}();

Tune tune() {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  return g_tune;
}

struct GemmCfg {
  int nblk = 0, ntblk = 0, splits = 1, tt = 1, ksteps = 0, K = 0, N = 0, depth = 2, kw = 1;
  size_t partial_floats() const { return gemm_partial_floats(nblk, splits, ntblk, tt); }
  size_t counters() const { return splits > 1 ? (size_t)nblk * ntblk : 0; }
};

// The wide streaming kernel: token blocks of 64 (T <= 64) or 128 tokens.
void set_wide(GemmCfg &c, int T, int splits) {
  c.kw = kGemmWide;
  c.tt = T <= 64 ? 4 : 8;
  c.ntblk = (T + 16 * c.tt - 1) / (16 * c.tt);
  c.splits = std::max(1, std::min(splits, c.ksteps));
}

// nblk: 32-row groups (16 gate/up feature pairs for SwiGLU).
// Enough row groups to fill the chip (2048 waves): one wave per unit, no K
// split, a shallow prefetch and many resident waves.  Too few: several waves
// of one workgroup per unit (4, 8 or 16, each at least 4 K steps), the fewest
// that reach 2048 waves; K split across units only if that is still short.
// The prefetch depth then covers a wave's steps in one or two rounds.
GemmCfg gemm_cfg(int kind, int nblk, int N, int T, int K, int wtype, bool packed) {
  constexpr int kFill = 2048;
  GemmCfg c;
  c.nblk = nblk;
  c.N = N;
  c.K = K;
  c.tt = T <= 16 ? 1 : T <= 32 ? 2 : T <= 48 ? 3 : 4;
  c.ntblk = (T + 16 * c.tt - 1) / (16 * c.tt);
  const int stream_tt = c.tt, stream_ntblk = c.ntblk;
  c.ksteps = K / kstep_of(wtype);
  const int base = std::max(1, nblk * c.ntblk);
  if (base >= kFill) {
    c.splits = 1;
    c.kw = 1;
    c.depth = 2;
  } else {
    const int wt = wtype == SV_W_BF16 ? WT_BF16 : wtype == SV_W_INT4_G32 ? WT_INT4 : WT_F32;
    for (int k : {4, 8, 16}) {
      if (c.ksteps / k < 4 || !gemm_kw_ok(wt, c.tt, k)) break;
      c.kw = k;
      if ((long long)base * k >= kFill) break;
    }
    const int waves = base * c.kw;
    if (waves < kFill) {
      const int room = std::max(1, c.ksteps / (4 * c.kw));
      c.splits = std::max(1, std::min(room, (kFill + waves - 1) / waves));
    }
    // 8 steps in flight take about 240 registers (2 waves per SIMD, 2048
    // resident): only when every wave is resident and has 8 steps to fetch
    const bool deep = gemm_deep_ok(wt, c.tt, c.kw);
    const long long nw = (long long)base * c.kw * c.splits;
    c.depth = deep && nw <= kFill && c.ksteps / (c.splits * c.kw) >= 8 ? 8 : 4;
    // at most two rounds of loads per wave while 4096 waves stay resident
    while (c.depth == 4 && c.ksteps / (c.splits * c.kw) > 8 &&
           (long long)base * c.kw * (c.splits + 1) <= 2 * kFill && c.ksteps / ((c.splits + 1) * c.kw) >= 4)
      ++c.splits;
    if ((kind == GK_O || kind == GK_DOWN) && c.kw > 4 && gemm_kw_ok(wt, c.tt, 4)) {
      // residual projections: four waves per unit and K splits to fill the chip
      // (measured 15-18% faster than 8 or 16 waves per unit sharing the K
      // range: the first wave's residual epilogue waits on a smaller reduction)
      c.kw = 4;
      const long long w4 = (long long)base * 4;
      c.splits = (int)std::max<long long>(1, std::min<long long>((kFill + w4 - 1) / w4, c.ksteps / 16));
      c.depth = 4;
    }
  }
  // many tokens (bf16, packed): the LDS-tiled kernel, when its grid of
  // (256 rows x 128 tokens) tiles has enough workgroups; from 49 tokens on it
  // beats streaming the head (measured), where the streaming kernel's
  // four-tile token blocks become bound by the token-operand traffic
  const bool tiled_ok = wtype == SV_W_BF16 && packed;
  const long long tiled_wgs = (long long)((nblk + 7) / 8) * ((T + 127) / 128);
  const long long square_wgs = (long long)((nblk + 7) / 8) * ((T + 255) / 256);
  // both kernels run one workgroup per CU; a 256 x 256 tile measured about
  // 1.75x the time of a 256 x 128 one (LM head, 1024 tokens: 129 vs 74 us per
  // round of 256 workgroups), so the square kernel wins when its rounds of
  // tiles take less time than the tiled kernel's
  const long long r_sq = (square_wgs + 255) / 256, r_t = (tiled_wgs + 255) / 256;
  if (tiled_ok && T >= 256 && 7 * r_sq < 4 * r_t) {
    // hundreds of tokens: the square-tiled kernel (the LM head from 512
    // tokens, gate||up from 384 at the 9B shape and 256 at the 27B one, QKV
    // at 2048; 27B-class gate||up at 256 tokens: 185 -> 161 us)
    c.kw = kGemmSquare;
    c.splits = 1;
  } else if (tiled_ok && T > 48 && tiled_wgs >= 256) {
    c.kw = kGemmTiled;
    c.splits = 1;
  } else if (tiled_ok && T > 48) {
    // too few tiles for the tiled kernel to fill the CUs: the wide streaming
    // kernel, with K splits filling one round of resident workgroups (one per
    // CU for 128-token blocks, two for 64), each split at least 8 K steps.
    // (The square kernel with K splits filling one round measured slower on
    // the 9B- and 27B-class QKV and O at 256 and 512 tokens: 65 -> 88 us for
    // O at 512; the partial tiles are 4 bytes per output per split.)
    set_wide(c, T, 1);
    const long long per = (long long)((nblk + 7) / 8) * c.ntblk;
    const long long slots = c.tt == 8 ? 256 : 512;
    c.splits = (int)std::max<long long>(1, std::min<long long>(slots / per, c.ksteps / 8));
    c.depth = 4;
  }
  const Tune tn = tune();
  if (tn.splits[kind] > 0) c.splits = std::max(1, std::min(tn.splits[kind], c.ksteps));
  if (tn.depth[kind] > 0) c.depth = tn.depth[kind];
  if (tn.kw[kind] == 0 && tiled_ok) {
    c.kw = kGemmTiled;
    c.splits = 1;
  } else if (tn.kw[kind] == 2 && tiled_ok && T > 16) {
    set_wide(c, T, tn.splits[kind] > 0 ? tn.splits[kind] : 1);
  } else if (tn.kw[kind] == 3 && tiled_ok) {
    c.kw = kGemmSquare;
    c.splits = tn.splits[kind] > 0 ? std::max(1, std::min(tn.splits[kind], c.ksteps / 2)) : 1;
  } else if (tn.kw[kind] > 0) {
    c.kw = tn.kw[kind] >= 16 ? 16 : tn.kw[kind] >= 8 ? 8 : tn.kw[kind] >= 4 ? 4 : 1;
  }
  if (c.kw == kGemmSquare && c.splits > 1) {  // partial tiles of 32 rows x 128 tokens
    c.tt = 8;
    c.ntblk = (T + 127) / 128;
  } else if (c.kw != kGemmWide) {  // the token blocking of the streaming kernels
    c.tt = stream_tt;
    c.ntblk = stream_ntblk;
  }
  if (c.kw == kGemmTiled) c.splits = 1;
  if (c.splits > 1 && (size_t)c.nblk * c.ntblk > kMaxCounters) c.splits = 1;
  return c;
}

// Packed int4 weights.  The int4 form of the wide streaming kernel shares
// each step's token fragments (through LDS) among the workgroup's 256 weight
// rows and converts each weight once per token block of 16, 32, 64 or 128
// tokens (in registers); K splits fill the resident workgroups (two per CU
// for blocks of up to 64 tokens, one for 128) at 4 or more int4 K steps each.
// From the size where the bf16 square-tiled kernel would win, its int4 form
// (converted in LDS).  The int4 streaming kernel (several waves per row
// group sharing K) stays where the wide grid is small: up to 64 tokens
// unless the matrix has 64 or more row blocks of 256 (the 9B-class LM head at
// 64 tokens: 390 -> 136 us, gate||up 69 -> 41 us; QKV and O slower), and up to
// 16 tokens unless it has 256 (the LM head: 94 -> 86 us).  Tuning overrides:
// waves per unit 1-16 keep the streaming int4 kernel, 2 (and 0: the tiled
// kernel has no int4 form) the wide one, 3 the square one.
GemmCfg gemm_cfg_w(int kind, int nblk, int N, int T, int K, int wtype, bool packed) {
  if (wtype == SV_W_INT4_G32 && packed) {
    const Tune tn = tune();
    const int ov = tn.kw[kind];
    if (ov == 1 || ov == 4 || ov == 8 || ov == 16) return gemm_cfg(kind, nblk, N, T, K, wtype, packed);
    GemmCfg b = gemm_cfg(kind, nblk, N, T, K, SV_W_BF16, true);
    if (b.kw == kGemmSquare && ov != 2 && ov != 0) return b;
    // the LM head from 129 to 256 tokens: one 256-token block of the square
    // kernel reads the weights once where the wide kernel's two 128-token
    // blocks read them twice (9B-class, 151936 rows: 160 tokens 414 -> 387 us,
    // 256 tokens 420 -> 411 us; from 257 the square kernel's half-empty second
    // block loses: 320 tokens 572 -> 673 us)
    if (kind == GK_HEAD && T > 128 && T <= 256 && ov < 0) {
      b.kw = kGemmSquare;
      b.splits = 1;
      return b;
    }
    GemmCfg c;
    c.nblk = nblk;
    c.N = N;
    c.K = K;
    c.ksteps = K / kstep_of(wtype);
    c.kw = kGemmWide;
    c.tt = T <= 16 ? 1 : T <= 32 ? 2 : T <= 64 ? 4 : 8;
    c.ntblk = (T + 16 * c.tt - 1) / (16 * c.tt);
    const long long per = (long long)((nblk + 7) / 8) * c.ntblk;
    const long long slots = c.tt == 8 ? 256 : 512;
    c.splits = (int)std::max<long long>(1, std::min<long long>(slots / per, c.ksteps / 4));
    if (tn.splits[kind] > 0) c.splits = std::max(1, std::min(tn.splits[kind], c.ksteps));
    c.depth = 2;
    if (c.splits > 1 && (size_t)c.nblk * c.ntblk > kMaxCounters) c.splits = 1;
    const int nrb = (nblk + 7) / 8;
    if (ov == 2 || ov == 0 || T > 64 || nrb >= (T > 16 ? 64 : 256)) return c;
  }
  return gemm_cfg(kind, nblk, N, T, K, wtype, packed);
}

// Token operands in fragment layout: the bf16 streaming launches with several
// waves per unit read them as contiguous KiB fragments (tiles = ntblk * tt).
bool frag_input(const GemmCfg &c, int wtype) {
  return wtype == SV_W_BF16 && (c.kw == 4 || c.kw == 8 || c.kw == 16);
}
int frag_tiles(const GemmCfg &c) { return c.ntblk * c.tt; }
size_t frag_bytes(const GemmCfg &c) { return (size_t)(c.K / 64) * frag_tiles(c) * 2048; }

struct LayerPlan {
  int T = 0, B = 0, G = 1, gmax = 0;
  GemmCfg qkv, o, gu, down, head;
  bool pk_qkv = false, pk_o = false, pk_gu = false, pk_down = false;
  size_t off_xp = 0, off_x1p = 0;
  int attn_chunk = 256, attn_items = 0, attn_rpad = 16;
  size_t off_counters = 0, off_partial = 0, off_qbuf = 0, off_po = 0, off_pml = 0;
  size_t off_attn = 0, off_x1 = 0, off_act = 0, off_stats = 0, off_items = 0;
  size_t off_rnorm = 0, off_rparts = 0, off_tseq = 0, off_tpos = 0, off_qs = 0, off_cs = 0, off_rope = 0;
  size_t off_tmask = 0, off_kvstage = 0;
  bool kv8 = false;
  size_t bytes = 0;
};

bool valid_wtype(int w) { return w == SV_W_F32 || w == SV_W_BF16 || w == SV_W_INT4_G32; }

sv_status check_matrix(const sv_matrix &m, int wtype) {
  if (!m.w) return SV_ERR_INVALID_ARG;
  if (wtype == SV_W_INT4_G32 && !m.scale) return SV_ERR_INVALID_ARG;
  return SV_OK;
}

sv_status plan_layer(const sv_layer *L, const sv_batch *b, int32_t flags, LayerPlan &pl) {
  if (!L || !b) return SV_ERR_INVALID_ARG;
  if (L->kind < SV_LAYER_EMBED || L->kind > SV_LAYER_HEAD) return SV_ERR_INVALID_ARG;
  if (flags & ~(SV_HEAD_LOGITS | SV_HEAD_LOGITS_STATS)) return SV_ERR_INVALID_ARG;
  if ((flags & SV_HEAD_LOGITS) && (flags & SV_HEAD_LOGITS_STATS)) return SV_ERR_INVALID_ARG;
  if (b->B < 0 || b->T < 0) return SV_ERR_INVALID_ARG;
  if (b->B > 0 && !b->gamma_host) return SV_ERR_INVALID_ARG;
  long long T = 0;
  int gmax = 0;
  for (int i = 0; i < b->B; ++i) {
    const int g = b->gamma_host[i];
    if (g < 0) return SV_ERR_INVALID_ARG;
    gmax = std::max(gmax, g);
    T += g + 1;
  }
  if (T != b->T) return SV_ERR_INVALID_ARG;
  if (T > (1 << 24)) return SV_ERR_UNSUPPORTED;
  pl.T = (int)T;
  pl.B = b->B;
  pl.gmax = gmax;
  if (L->d <= 0) return SV_ERR_INVALID_ARG;
  if (pl.T == 0) {  // empty batch: nothing to plan, nothing will be enqueued
    pl.bytes = 0;
    return SV_OK;
  }
  const int w = L->wtype;
  const bool packed = L->layout == SV_LAYOUT_PACKED;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };

  if (L->kind == SV_LAYER_EMBED) {
    if (L->vocab <= 0 || !L->embed.w) return SV_ERR_INVALID_ARG;
    if (w != SV_W_F32 && w != SV_W_BF16) return SV_ERR_UNSUPPORTED;
    pl.bytes = 0;
    return SV_OK;
  }
  if (!valid_wtype(w)) return SV_ERR_UNSUPPORTED;
  if (L->layout != SV_LAYOUT_ROWMAJOR && L->layout != SV_LAYOUT_PACKED) return SV_ERR_INVALID_ARG;
  if (L->layout == SV_LAYOUT_PACKED && w == SV_W_F32) return SV_ERR_UNSUPPORTED;
  const int kmul = w == SV_W_INT4_G32 ? 128 : 64;
  if (L->d % kmul) return SV_ERR_UNSUPPORTED;

  if (L->kind == SV_LAYER_HEAD) {
    if (L->vocab <= 0) return SV_ERR_INVALID_ARG;
    if (check_matrix(L->lm_head, w) != SV_OK) return SV_ERR_INVALID_ARG;
    pl.head = gemm_cfg_w(GK_HEAD, (L->vocab + 31) / 32, L->vocab, pl.T, L->d, w, packed);
    pl.off_counters = take(kCounterBytes);
    pl.off_partial = take(pl.head.partial_floats() * sizeof(float));
    pl.off_stats = take((size_t)pl.head.nblk * pl.T * 2 * sizeof(float));
    pl.off_rnorm = take((size_t)pl.T * sizeof(float));
    pl.bytes = off;
    return SV_OK;
  }

  // DECODER
  const int d = L->d, hq = L->n_q_heads, hk = L->n_kv_heads, hd = L->head_dim, F = L->ffn;
  if (hq <= 0 || hk <= 0 || F <= 0) return SV_ERR_INVALID_ARG;
  if (hq % hk) return SV_ERR_UNSUPPORTED;
  if (hd != 64 && hd != 128) return SV_ERR_UNSUPPORTED;
  if (F % kmul || (hq * hd) % kmul) return SV_ERR_UNSUPPORTED;
  for (const sv_matrix *m : {&L->wq, &L->wk, &L->wv, &L->wo, &L->w_gate, &L->w_up, &L->w_down})
    if (check_matrix(*m, w) != SV_OK) return SV_ERR_INVALID_ARG;
  pl.G = hq / hk;
  if (pl.B > kScanMaxB) return SV_ERR_UNSUPPORTED;
  if ((long long)pl.G * (gmax + 1) > kAttnMaxRows) return SV_ERR_UNSUPPORTED;
  // token trees: every tree within the 64-node ancestor masks
  if (b->tree_parent && gmax + 1 > kMaxTreeNodes) return SV_ERR_UNSUPPORTED;
  // int8 caches: codes plus per-vector scales (both attention kernels)
  if (b->kv_dtype != SV_KV_BF16 && b->kv_dtype != SV_KV_INT8) return SV_ERR_INVALID_ARG;
  pl.kv8 = b->kv_dtype == SV_KV_INT8;
  if (pl.kv8 && pl.B > 0 && (!b->k_scale || !b->v_scale)) return SV_ERR_INVALID_ARG;
  // per-sequence capacity (kv_len[i] + gamma_i + 1 <= kv_cap) is checked on the
  // device, where kv_len lives; max_ctx only sizes the attention grid
  if (b->max_ctx < 0 || b->kv_cap <= 0 || b->kv_cap % 32) return SV_ERR_INVALID_ARG;
  if ((long long)pl.B * hk > (long long)kMaxCounters) return SV_ERR_UNSUPPORTED;
  if (pl.B > 0 && (!b->gamma || !b->kv_len || !b->k_cache || !b->v_cache)) return SV_ERR_INVALID_ARG;

  const int nqkv = (hq + 2 * hk) * hd;
  pl.qkv = gemm_cfg_w(GK_QKV, nqkv / 32, nqkv, pl.T, d, w, packed);
  pl.o = gemm_cfg_w(GK_O, (d + 31) / 32, d, pl.T, hq * hd, w, packed);
  pl.gu = gemm_cfg_w(GK_GU, (F + 15) / 16, 2 * F, pl.T, d, w, packed);
  pl.down = gemm_cfg_w(GK_DOWN, (d + 31) / 32, d, pl.T, F, w, packed);
  pl.attn_rpad = 16 * ((pl.G * (gmax + 1) + 15) / 16);
  // keys per work item (a multiple of 128): enough items for two workgroups
  // per CU at hd 128 (three fit -- the key-split kernel holds a step's keys
  // and values in registers at once, the query-tiled one 48 KiB of LDS -- but
  // the third's shorter chunks and extra merge inputs cost more than its
  // loads in flight gain: 86 -> 82 us at 256 query tokens and 2048 cached,
  // 25.0 -> 23.2 us at 24 tokens), 4 at hd 64, and at least 256 keys and
  // ceil(length / 32) (a sequence has at most 32)
  const long long max_len = (long long)b->max_ctx + gmax + 1;
  const long long slots = 256LL * (hd == 64 ? 4 : 2);
  const long long per_seq = std::max<long long>(1, slots / std::max<long long>(1, (long long)pl.B * hk));
  long long chunk = (max_len + per_seq - 1) / per_seq;
  chunk = std::max({chunk, 256LL, (max_len + 31) / 32});
  pl.attn_chunk = (int)((chunk + 127) / 128 * 128);
  long long items = 0;
  for (int i = 0; i < pl.B; ++i)
    items += ((long long)b->max_ctx + b->gamma_host[i] + 1 + pl.attn_chunk - 1) / pl.attn_chunk;
  if (items > (1 << 30)) return SV_ERR_UNSUPPORTED;
  pl.attn_items = (int)items;

  pl.pk_qkv = frag_input(pl.qkv, w);
  pl.pk_o = frag_input(pl.o, w);
  pl.pk_gu = frag_input(pl.gu, w);
  pl.pk_down = frag_input(pl.down, w);
  size_t partial = 0;
  for (const GemmCfg *g : {&pl.qkv, &pl.o, &pl.gu, &pl.down}) partial = std::max(partial, g->partial_floats());
  pl.off_counters = take(kCounterBytes);
  pl.off_partial = take(partial * sizeof(float));
  pl.off_qbuf = take((size_t)pl.T * hq * hd * 2);
  pl.off_po = take((size_t)pl.attn_items * hk * pl.attn_rpad * hd * sizeof(float));
  pl.off_pml = take((size_t)pl.attn_items * hk * pl.attn_rpad * 2 * sizeof(float));
  pl.off_attn = take(std::max((size_t)pl.T * hq * hd * 2, pl.pk_o ? frag_bytes(pl.o) : 0));
  pl.off_x1 = take((size_t)pl.T * d * 2);
  pl.off_act = take(std::max((size_t)pl.T * F * 2, pl.pk_down ? frag_bytes(pl.down) : 0));
  pl.off_xp = take(pl.pk_qkv ? frag_bytes(pl.qkv) : 0);
  pl.off_x1p = take(pl.pk_gu ? frag_bytes(pl.gu) : 0);
  // one buffer for the dequantised weights of whichever projection runs
  pl.off_rnorm = take((size_t)pl.T * sizeof(float));
  pl.off_rparts = take((size_t)pl.o.nblk * pl.T * sizeof(float));
  pl.off_tseq = take((size_t)pl.T * sizeof(int));
  pl.off_tpos = take((size_t)pl.T * sizeof(int));
  pl.off_tmask = take(b->tree_parent ? (size_t)pl.T * sizeof(unsigned long long) : 0);
  pl.off_kvstage = take(pl.kv8 ? (size_t)pl.T * 2 * hk * hd * 2 : 0);
  pl.off_qs = take((size_t)(pl.B + 1) * sizeof(int));
  pl.off_cs = take((size_t)(pl.B + 1) * sizeof(int));
  pl.off_items = take((size_t)pl.attn_items * 2 * sizeof(int4));
  pl.off_rope = take((size_t)pl.T * hd * sizeof(float));
  pl.bytes = off;
  return SV_OK;
}

GemmParams base_params(const GemmCfg &c, const void *x, int T, int wtype, unsigned char *ws,
                       const LayerPlan &pl) {
  GemmParams p;
  std::memset(&p, 0, sizeof(p));
  p.x = static_cast<const uint16_t *>(x);
  p.T = T;
  p.K = c.K;
  p.N = c.N;
  p.splits = c.splits;
  p.ksteps = c.ksteps;
  p.nblk = c.nblk;
  p.ntblk = c.ntblk;
  p.packed = 0;
  p.partial = reinterpret_cast<float *>(ws + pl.off_partial);
  p.counters = reinterpret_cast<int *>(ws + pl.off_counters);
  (void)wtype;
  return p;
}

int wt_of(int w) { return w == SV_W_F32 ? WT_F32 : w == SV_W_BF16 ? WT_BF16 : WT_INT4; }

GemmMat mat_of(const sv_matrix &m, int rows) {
  GemmMat g;
  g.w = m.w;
  g.s = static_cast<const uint16_t *>(m.scale);
  g.rows = rows;
  return g;
}

}  // namespace

extern "C" sv_status sv_verify_layer_workspace_bytes(const sv_layer *layer, const sv_batch *batch,
                                                     int32_t flags, size_t *bytes) {
  if (!bytes) return SV_ERR_INVALID_ARG;
  LayerPlan pl;
  const sv_status st = plan_layer(layer, batch, flags, pl);
  if (st != SV_OK) return st;
  *bytes = pl.bytes;
  return SV_OK;
}

extern "C" sv_status sv_verify_layer(const sv_layer *L, const sv_batch *b, const void *x_in,
                                     void *y_out, int32_t flags, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  LayerPlan pl;
  sv_status st = plan_layer(L, b, flags, pl);
  if (st != SV_OK) return st;
  if (pl.T == 0) return SV_OK;
  if (!x_in || !y_out) return SV_ERR_INVALID_ARG;
  if (pl.bytes > 0 && (!workspace || workspace_bytes < pl.bytes)) return SV_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  const int wt = wt_of(L->wtype);
  (void)hipGetLastError();  // start from a clean launch status
  hipError_t e = hipSuccess;

  if (L->kind == SV_LAYER_EMBED) {
    EmbedParams p;
    p.tokens = static_cast<const int *>(x_in);
    p.table = L->embed.w;
    p.table_bf16 = L->wtype == SV_W_BF16;
    p.T = pl.T;
    p.V = L->vocab;
    p.d = L->d;
    p.out = static_cast<uint16_t *>(y_out);
    p.err = b->err_flag;
    e = launch_embed(p, s);
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
  }

  if (L->kind == SV_LAYER_HEAD) {
    GemmParams p = base_params(pl.head, x_in, pl.T, wt, ws, pl);
    if (pl.head.kw == 1 && pl.head.splits == 1) {
      // one wave per unit, whole K range: the kernel takes the RMSNorm scale
      // from the token rows it loads (no separate pass)
      p.rms_inline = 1;
    } else {
      PrepParams pp;
      std::memset(&pp, 0, sizeof(pp));
      pp.x = static_cast<const uint16_t *>(x_in);
      pp.T = pl.T;
      pp.d = L->d;
      pp.eps = L->eps;
      pp.rnorm = reinterpret_cast<float *>(ws + pl.off_rnorm);
      e = launch_prep(pp, s);
      if (e != hipSuccess) return SV_ERR_HIP;
      p.rnorm = pp.rnorm;
    }
    p.packed = L->layout == SV_LAYOUT_PACKED;
    p.nmat = 1;
    p.mat[0] = mat_of(L->lm_head, L->vocab);
    p.rowmap = RM_LINEAR;
    p.eps = L->eps;
    p.epi = EPI_LOGITS;
    p.out = y_out;
    p.ldo = L->vocab;
    p.stats = reinterpret_cast<float *>(ws + pl.off_stats);
    const int wl = wt;
    e = launch_gemm(p, wl, pl.head.tt, pl.head.depth, pl.head.kw, s, SV_K_GEMM_LM_HEAD);
    if (e == hipSuccess && !(flags & SV_HEAD_LOGITS)) {
      HeadSoftmaxParams h;
      h.logits = static_cast<float *>(y_out);
      h.stats = p.stats;
      h.T = pl.T;
      h.V = L->vocab;
      h.nblk = pl.head.nblk;
      h.cols_per_block = kSoftmaxCols;
      h.row_ms = static_cast<float *>(y_out) + (size_t)pl.T * L->vocab;
      e = (flags & SV_HEAD_LOGITS_STATS) ? launch_head_rowstats(h, s) : launch_head_softmax(h, s);
    }
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
  }

  // DECODER
  const int d = L->d, hq = L->n_q_heads, hk = L->n_kv_heads, hd = L->head_dim, F = L->ffn;
  uint16_t *qbuf = reinterpret_cast<uint16_t *>(ws + pl.off_qbuf);
  uint16_t *attn = reinterpret_cast<uint16_t *>(ws + pl.off_attn);
  uint16_t *x1 = reinterpret_cast<uint16_t *>(ws + pl.off_x1);
  uint16_t *act = reinterpret_cast<uint16_t *>(ws + pl.off_act);

  float *rnorm = reinterpret_cast<float *>(ws + pl.off_rnorm);
  float *rparts = reinterpret_cast<float *>(ws + pl.off_rparts);
  int *tseq = reinterpret_cast<int *>(ws + pl.off_tseq);
  int *tpos = reinterpret_cast<int *>(ws + pl.off_tpos);
  int *qstart = reinterpret_cast<int *>(ws + pl.off_qs);
  int *cstart = reinterpret_cast<int *>(ws + pl.off_cs);
  {  // RMSNorm scales of x and the token map
    PrepParams pp;
    std::memset(&pp, 0, sizeof(pp));
    pp.x = static_cast<const uint16_t *>(x_in);
    pp.T = pl.T;
    pp.d = d;
    pp.eps = L->eps;
    pp.rnorm = rnorm;
    pp.gamma = b->gamma;
    pp.kv_len = b->kv_len;
    pp.B = pl.B;
    pp.chunk = pl.attn_chunk;
    pp.tok_seq = tseq;
    pp.tok_pos = tpos;
    pp.q_start = qstart;
    pp.chunk_start = cstart;
    pp.rope_cs = reinterpret_cast<float *>(ws + pl.off_rope);
    pp.hd = hd;
    pp.tree_parent = b->tree_parent;
    pp.tree_mask = b->tree_parent ? reinterpret_cast<unsigned long long *>(ws + pl.off_tmask) : nullptr;
    pp.items = reinterpret_cast<int4 *>(ws + pl.off_items);
    pp.max_items = pl.attn_items;
    pp.max_ctx = b->max_ctx;
    pp.xp = pl.pk_qkv ? reinterpret_cast<uint16_t *>(ws + pl.off_xp) : nullptr;
    pp.xp_ntt = frag_tiles(pl.qkv);
    pp.err = b->err_flag;
    for (int i = 0; i < hd / 2; ++i)
      pp.inv_freq[i] = std::pow(static_cast<double>(L->rope_theta), -2.0 * i / hd);
    e = launch_prep(pp, s);
    if (e != hipSuccess) return SV_ERR_HIP;
  }
  {  // QKV + RoPE + KV append
    GemmParams p = base_params(pl.qkv, x_in, pl.T, wt, ws, pl);
    if (pl.pk_qkv) {
      p.xp = reinterpret_cast<const uint16_t *>(ws + pl.off_xp);
      p.xp_ntt = frag_tiles(pl.qkv);
    }
    p.rnorm = rnorm;
    p.packed = L->layout == SV_LAYOUT_PACKED;
    p.nmat = 3;
    p.mat[0] = mat_of(L->wq, hq * hd);
    p.mat[1] = mat_of(L->wk, hk * hd);
    p.mat[2] = mat_of(L->wv, hk * hd);
    p.rowmap = RM_ROPE_PAIRS;
    p.hd = hd;
    p.eps = L->eps;
    p.epi = EPI_QKV;
    p.qbuf = qbuf;
    p.hq = hq;
    p.hkv = hk;
    p.tok_seq = tseq;
    p.tok_pos = tpos;
    p.rope_cs = reinterpret_cast<const float *>(ws + pl.off_rope);
    p.B = pl.B;
    p.kv_cap = b->kv_cap;
    p.kc = b->k_cache;
    p.vc = b->v_cache;
    p.kvstage = pl.kv8 ? reinterpret_cast<uint16_t *>(ws + pl.off_kvstage) : nullptr;
    p.err = b->err_flag;
    const int wl = wt;
    e = launch_gemm(p, wl, pl.qkv.tt, pl.qkv.depth, pl.qkv.kw, s, SV_K_GEMM_QKV);
    if (e != hipSuccess) return SV_ERR_HIP;
  }
  if (pl.kv8) {  // the new keys and values into the int8 caches
    KvQuantParams q;
    q.kvstage = reinterpret_cast<const uint16_t *>(ws + pl.off_kvstage);
    q.tok_seq = tseq;
    q.tok_pos = tpos;
    q.T = pl.T;
    q.hkv = hk;
    q.hd = hd;
    q.kv_cap = b->kv_cap;
    q.kc = b->k_cache;
    q.vc = b->v_cache;
    q.ksc = b->k_scale;
    q.vsc = b->v_scale;
    e = launch_kv_quant(q, s);
    if (e != hipSuccess) return SV_ERR_HIP;
  }
  {  // ragged attention (chunks merged by the last to arrive)
    AttnParams a;
    std::memset(&a, 0, sizeof(a));
    a.qbuf = qbuf;
    a.items = reinterpret_cast<const int4 *>(ws + pl.off_items);
    a.kc = b->k_cache;
    a.vc = b->v_cache;
    a.B = pl.B;
    a.T = pl.T;
    a.hq = hq;
    a.hkv = hk;
    a.hd = hd;
    a.kv_cap = b->kv_cap;
    a.max_ctx = b->max_ctx;
    a.tree_mask = b->tree_parent ? reinterpret_cast<const unsigned long long *>(ws + pl.off_tmask) : nullptr;
    a.kv8 = pl.kv8 ? 1 : 0;
    a.ksc = b->k_scale;
    a.vsc = b->v_scale;
    a.chunk = pl.attn_chunk;
    a.max_items = pl.attn_items;
    a.rpad = pl.attn_rpad;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)hd));
    a.part_o = reinterpret_cast<float *>(ws + pl.off_po);
    a.part_ml = reinterpret_cast<float *>(ws + pl.off_pml);
    a.out = attn;
    a.out_ntt = pl.pk_o ? frag_tiles(pl.o) : 0;
    a.counters = reinterpret_cast<int *>(ws + pl.off_counters);
    a.err = b->err_flag;
    e = launch_attention(a, s);
    if (e != hipSuccess) return SV_ERR_HIP;
  }
  {  // O projection + residual
    GemmParams p = base_params(pl.o, attn, pl.T, wt, ws, pl);
    if (pl.pk_o) {
      p.xp = attn;
      p.xp_ntt = frag_tiles(pl.o);
    }
    if (pl.pk_gu) {  // the gate||up token operand, besides x1 itself
      p.out_pk = reinterpret_cast<uint16_t *>(ws + pl.off_x1p);
      p.out_pk_ntt = frag_tiles(pl.gu);
    }
    p.packed = L->layout == SV_LAYOUT_PACKED;
    p.nmat = 1;
    p.mat[0] = mat_of(L->wo, d);
    p.rowmap = RM_LINEAR;
    p.epi = EPI_RESID;
    p.out = x1;
    p.ldo = d;
    p.resid = static_cast<const uint16_t *>(x_in);
    p.sq_out = rparts;  // sums of squares of x1 for the next RMSNorm
    const int wl = wt;
    e = launch_gemm(p, wl, pl.o.tt, pl.o.depth, pl.o.kw, s, SV_K_GEMM_O);
    if (e != hipSuccess) return SV_ERR_HIP;
  }
  {  // gate || up + SwiGLU
    GemmParams p = base_params(pl.gu, x1, pl.T, wt, ws, pl);
    if (pl.pk_gu) {
      p.xp = reinterpret_cast<const uint16_t *>(ws + pl.off_x1p);
      p.xp_ntt = frag_tiles(pl.gu);
    }
    if (pl.pk_down) {  // act only feeds the down projection
      p.out_pk = act;
      p.out_pk_ntt = frag_tiles(pl.down);
    }
    p.packed = L->layout == SV_LAYOUT_PACKED;
    p.nmat = 2;
    p.mat[0] = mat_of(L->w_gate, F);
    p.mat[1] = mat_of(L->w_up, F);
    p.rowmap = RM_SWIGLU;
    if (rs_parts_in_gemm(pl.gu.kw, pl.gu.tt, pl.o.nblk)) {
      p.rparts = rparts;  // staged in LDS by the GEMM itself
      p.nparts = pl.o.nblk;
    } else {
      // one scale per token first (the tiled kernels would otherwise gather the
      // partials once per lane and token tile)
      e = launch_rnorm_parts(rparts, pl.o.nblk, pl.T, d, L->eps, rnorm, s);
      if (e != hipSuccess) return SV_ERR_HIP;
      p.rnorm = rnorm;
    }
    p.eps = L->eps;
    p.epi = EPI_SWIGLU;
    p.out = act;
    p.ldo = F;
    const int wl = wt;
    e = launch_gemm(p, wl, pl.gu.tt, pl.gu.depth, pl.gu.kw, s, SV_K_GEMM_GATE_UP);
    if (e != hipSuccess) return SV_ERR_HIP;
  }
  {  // down projection + residual
    GemmParams p = base_params(pl.down, act, pl.T, wt, ws, pl);
    if (pl.pk_down) {
      p.xp = act;
      p.xp_ntt = frag_tiles(pl.down);
    }
    p.packed = L->layout == SV_LAYOUT_PACKED;
    p.nmat = 1;
    p.mat[0] = mat_of(L->w_down, d);
    p.rowmap = RM_LINEAR;
    p.epi = EPI_RESID;
    p.out = y_out;
    p.ldo = d;
    p.resid = x1;
    const int wl = wt;
    e = launch_gemm(p, wl, pl.down.tt, pl.down.depth, pl.down.kw, s, SV_K_GEMM_DOWN);
    if (e != hipSuccess) return SV_ERR_HIP;
  }
  return SV_OK;
}

// ---------------------------------------------------------------------------
// Packed weight layout.
extern "C" sv_status sv_packed_matrix_bytes(int32_t wtype, int32_t N, int32_t K, size_t *w_bytes,
                                            size_t *scale_bytes) {
  if (N <= 0 || K <= 0) return SV_ERR_INVALID_ARG;
  const size_t rows = (size_t)(N + 31) / 32 * 32;
  if (wtype == SV_W_BF16) {
    if (K % 64) return SV_ERR_UNSUPPORTED;
    if (w_bytes) *w_bytes = rows * K * 2;
    if (scale_bytes) *scale_bytes = 0;
    return SV_OK;
  }
  if (wtype == SV_W_INT4_G32) {
    if (K % 128) return SV_ERR_UNSUPPORTED;
    if (w_bytes) *w_bytes = rows * K / 2;
    if (scale_bytes) *scale_bytes = rows * (K / 32) * 2;
    return SV_OK;
  }
  return SV_ERR_UNSUPPORTED;
}

extern "C" sv_status sv_pack_matrix(int32_t wtype, int32_t N, int32_t K, const void *w,
                                    const void *scale, void *w_packed, void *scale_packed,
                                    void *stream) {
  size_t wb = 0, sb = 0;
  const sv_status st = sv_packed_matrix_bytes(wtype, N, K, &wb, &sb);
  if (st != SV_OK) return st;
  if (!w || !w_packed) return SV_ERR_INVALID_ARG;
  if (wtype == SV_W_INT4_G32 && (!scale || !scale_packed)) return SV_ERR_INVALID_ARG;
  (void)hipGetLastError();
  const hipError_t e = launch_pack(wtype == SV_W_BF16 ? WT_BF16 : WT_INT4, N, K, w, scale, w_packed,
                                   scale_packed, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Acceptance.
namespace {
// Vocabulary chunk per workgroup: 4096 entries, or 8192 once the batch has
// more than about 1024 workgroups' worth of chunks, where each workgroup's
// latency chain is better spent on twice the loads (measured: 77 -> 67 us at
// B = 128, 16.7 -> 18.8 us at B = 8; 2048-entry chunks at B = 8: 16.8 ->
// 19.9 us).
constexpr int kAcceptChunk = 4096;
constexpr int kAcceptChunkWide = 8192;

}  // namespace

// counter_bytes: room for the per-sequence arrival counters at the start of
// the scratch memory (the shared workspace layout reserves kCounterBytes).
sv_status sv::plan_accept(int32_t B, int32_t V, int32_t mode, const int32_t *gamma_host, AcceptPlan &ap,
                      size_t counter_bytes) {
  if (B < 0 || V <= 0) return SV_ERR_INVALID_ARG;
  if (mode & ~(0xFF | SV_ACCEPT_FROM_LOGITS)) return SV_ERR_INVALID_ARG;
  mode &= 0xFF;
  if (mode != SV_ACCEPT_STOCHASTIC && mode != SV_ACCEPT_GREEDY) return SV_ERR_INVALID_ARG;
  if (B > 0 && !gamma_host) return SV_ERR_INVALID_ARG;
  if (B > kScanMaxB) return SV_ERR_UNSUPPORTED;
  for (int i = 0; i < B; ++i) {
    if (gamma_host[i] < 0) return SV_ERR_INVALID_ARG;
    ap.T += gamma_host[i] + 1;
    ap.nd += gamma_host[i];
  }
  if (ap.T > (1 << 24)) return SV_ERR_UNSUPPORTED;
  ap.chunk = (long long)B * ((V + kAcceptChunk - 1) / kAcceptChunk) > 1024 ? kAcceptChunkWide : kAcceptChunk;
  ap.nchunk = (V + ap.chunk - 1) / ap.chunk;
  const long long rows = mode == SV_ACCEPT_GREEDY ? ap.T : B;
  size_t off = counter_bytes;  // counters first
  ap.off_parts = off;
  off = align_up(off + (size_t)rows * ap.nchunk * sizeof(AcceptPart));
  ap.off_acc = off;
  off = align_up(off + (size_t)(B + ap.T) * sizeof(int));
  ap.bytes = off;
  return SV_OK;
}

extern "C" sv_status sv_accept_commit_workspace_bytes(int32_t B, int32_t V, int32_t mode,
                                                      const int32_t *gamma_host, size_t *bytes) {
  if (!bytes) return SV_ERR_INVALID_ARG;
  AcceptPlan ap;
  const sv_status st = plan_accept(B, V, mode, gamma_host, ap, kCounterBytes);
  if (st != SV_OK) return st;
  *bytes = ap.bytes;
  return SV_OK;
}

// Host checks of an acceptance call's pointers (after plan_accept).
sv_status sv::check_accept_args(int32_t B, int32_t mode, const AcceptPlan &ap, const int32_t *gamma,
                            const int32_t *draft, const float *p, const float *q, const float *u_acc,
                            const float *u_samp, const int32_t *kv_len, const int32_t *accepted,
                            const int32_t *next_token) {
  if (B == 0) return SV_OK;
  if (!gamma || !p || !kv_len || !accepted || !next_token) return SV_ERR_INVALID_ARG;
  if (ap.nd > 0 && !draft) return SV_ERR_INVALID_ARG;
  if ((mode & 0xFF) == SV_ACCEPT_STOCHASTIC) {
    if (!u_samp) return SV_ERR_INVALID_ARG;
    if (ap.nd > 0 && (!q || !u_acc)) return SV_ERR_INVALID_ARG;
  }
  return SV_OK;
}

// Enqueue the acceptance kernel with its scratch memory at ws (counters at
// ws, zero on entry; the rest at the plan's offsets).
sv_status sv::run_accept(int32_t B, int32_t V, int32_t mode, const int32_t *gamma_host, const AcceptPlan &ap,
                     const int32_t *gamma, const int32_t *draft, const float *p, const float *q,
                     const float *u_acc, const float *u_samp, int32_t *kv_len, int32_t *accepted,
                     int32_t *next_token, int32_t *err_flag, unsigned char *ws, hipStream_t stream) {
  const bool from_logits = (mode & SV_ACCEPT_FROM_LOGITS) != 0;
  AcceptParams a;
  std::memset(&a, 0, sizeof(a));
  a.B = B;
  a.V = V;
  a.T = (int)ap.T;
  a.nd = (int)ap.nd;
  a.mode = mode & 0xFF;
  a.chunk = ap.chunk;
  a.nchunk = ap.nchunk;
  a.gamma = gamma;
  a.draft = draft;
  a.p = p;
  a.row_ms = from_logits ? p + ap.T * (size_t)V : nullptr;
  a.q = q;
  a.u_acc = u_acc;
  a.u_samp = u_samp;
  a.kv_len = kv_len;
  a.accepted = accepted;
  a.next_token = next_token;
  a.err = err_flag;
  a.parts = reinterpret_cast<AcceptPart *>(ws + ap.off_parts);
  a.acc_ws = reinterpret_cast<int *>(ws + ap.off_acc);
  a.counters = reinterpret_cast<int *>(ws);
  if (B <= kAcceptHostMax) {
    a.host_map = 1;
    int qs = 0;
    for (int i = 0; i < B; ++i) {
      a.hq_start[i] = qs;
      a.hgamma[i] = gamma_host[i];
      qs += gamma_host[i] + 1;
    }
  }
  const hipError_t e = launch_accept(a, stream);
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

extern "C" sv_status sv_accept_commit(int32_t B, int32_t V, int32_t mode, const int32_t *gamma_host,
                                      const int32_t *gamma, const int32_t *draft, const float *p,
                                      const float *q, const float *u_acc, const float *u_samp,
                                      int32_t *kv_len, int32_t *accepted, int32_t *next_token,
                                      int32_t *err_flag, void *workspace, size_t workspace_bytes,
                                      void *stream) {
  AcceptPlan ap;
  sv_status st = plan_accept(B, V, mode, gamma_host, ap, kCounterBytes);
  if (st != SV_OK) return st;
  st = check_accept_args(B, mode, ap, gamma, draft, p, q, u_acc, u_samp, kv_len, accepted, next_token);
  if (st != SV_OK || B == 0) return st;
  if (!workspace || workspace_bytes < ap.bytes) return SV_ERR_WORKSPACE;
  (void)hipGetLastError();
  return run_accept(B, V, mode, gamma_host, ap, gamma, draft, p, q, u_acc, u_samp, kv_len, accepted,
                    next_token, err_flag, static_cast<unsigned char *>(workspace),
                    static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// Token trees.
namespace {
sv_status plan_tree(int32_t B, int32_t V, const int32_t *gamma_host, long long &T, size_t &bytes) {
  if (B < 0 || V <= 0 || (B > 0 && !gamma_host)) return SV_ERR_INVALID_ARG;
  if (B > kTreeMaxB) return SV_ERR_UNSUPPORTED;
  T = 0;
  for (int i = 0; i < B; ++i) {
    if (gamma_host[i] < 0) return SV_ERR_INVALID_ARG;
    if (gamma_host[i] + 1 > kMaxTreeNodes) return SV_ERR_UNSUPPORTED;
    T += gamma_host[i] + 1;
  }
  bytes = tree_workspace_bytes(B, V, T);
  return SV_OK;
}
}  // namespace

extern "C" sv_status sv_accept_tree_workspace_bytes(int32_t B, int32_t V, const int32_t *gamma_host,
                                                    size_t *bytes) {
  if (!bytes) return SV_ERR_INVALID_ARG;
  long long T = 0;
  return plan_tree(B, V, gamma_host, T, *bytes);
}

extern "C" sv_status sv_accept_tree(int32_t B, int32_t V, int32_t mode, const int32_t *gamma_host,
                                    const int32_t *parent, const int32_t *tokens, const float *p,
                                    const float *q, const float *u_acc, const float *u_samp,
                                    int32_t *kv_len, int32_t *accepted, int32_t *next_token, int32_t *path,
                                    int32_t *err_flag, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  const bool from_logits = (mode & SV_ACCEPT_FROM_LOGITS) != 0;
  mode &= ~SV_ACCEPT_FROM_LOGITS;
  if (mode != SV_ACCEPT_STOCHASTIC && mode != SV_ACCEPT_GREEDY) return SV_ERR_INVALID_ARG;
  long long T = 0;
  size_t bytes = 0;
  sv_status st = plan_tree(B, V, gamma_host, T, bytes);
  if (st != SV_OK || B == 0) return st;
  if (!parent || !tokens || !p || !kv_len || !accepted || !next_token || !path) return SV_ERR_INVALID_ARG;
  if (mode == SV_ACCEPT_STOCHASTIC && (!q || !u_acc || !u_samp)) return SV_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < bytes) return SV_ERR_WORKSPACE;
  TreeAcceptParams a;
  std::memset(&a, 0, sizeof(a));
  a.B = B;
  a.V = V;
  a.greedy = mode == SV_ACCEPT_GREEDY;
  a.parent = parent;
  a.tokens = tokens;
  a.p = p;
  a.row_ms = from_logits ? p + (size_t)T * V : nullptr;
  a.q = q;
  a.u_acc = u_acc;
  a.u_samp = u_samp;
  a.kv_len = kv_len;
  a.accepted = accepted;
  a.next_token = next_token;
  a.path = path;
  a.err = err_flag;
  a.ws = static_cast<unsigned char *>(workspace);
  int qs = 0;
  for (int i = 0; i < B; ++i) {
    a.q_start[i] = qs;
    qs += gamma_host[i] + 1;
  }
  a.q_start[B] = qs;
  (void)hipGetLastError();
  return launch_tree_accept(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

namespace {
sv_status tree_commit(int32_t B, int32_t n_kv_heads, int32_t head_dim, int32_t kv_cap, const int32_t *kv_len,
                      const int32_t *accepted, const int32_t *path, void *const *k_cache, void *const *v_cache,
                      void *const *k_scale, void *const *v_scale, void *stream) {
  if (B < 0 || n_kv_heads <= 0 || head_dim <= 0 || kv_cap <= 0 || kv_cap % 32) return SV_ERR_INVALID_ARG;
  if (B == 0) return SV_OK;
  if (!kv_len || !accepted || !path || !k_cache || !v_cache) return SV_ERR_INVALID_ARG;
  TreeCommitParams c;
  c.kv8 = k_scale != nullptr;
  c.ksc = k_scale;
  c.vsc = v_scale;
  c.B = B;
  c.hkv = n_kv_heads;
  c.hd = head_dim;
  c.kv_cap = kv_cap;
  c.kv_len = kv_len;
  c.accepted = accepted;
  c.path = path;
  c.kc = k_cache;
  c.vc = v_cache;
  (void)hipGetLastError();
  return launch_tree_commit(c, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}
}  // namespace

extern "C" sv_status sv_tree_commit_kv(int32_t B, int32_t n_kv_heads, int32_t head_dim, int32_t kv_cap,
                                       const int32_t *kv_len, const int32_t *accepted, const int32_t *path,
                                       void *const *k_cache, void *const *v_cache, void *stream) {
  return tree_commit(B, n_kv_heads, head_dim, kv_cap, kv_len, accepted, path, k_cache, v_cache, nullptr, nullptr,
                     stream);
}

extern "C" sv_status sv_tree_commit_kv_int8(int32_t B, int32_t n_kv_heads, int32_t head_dim, int32_t kv_cap,
                                            const int32_t *kv_len, const int32_t *accepted, const int32_t *path,
                                            void *const *k_cache, void *const *v_cache, void *const *k_scale,
                                            void *const *v_scale, void *stream) {
  if (B > 0 && (!k_scale || !v_scale)) return SV_ERR_INVALID_ARG;
  return tree_commit(B, n_kv_heads, head_dim, kv_cap, kv_len, accepted, path, k_cache, v_cache, k_scale, v_scale,
                     stream);
}

extern "C" sv_status sv_accept_position_counts(int32_t B, int32_t n_pos, const int32_t *gamma,
                                               const int32_t *accepted, int64_t *counts, void *stream) {
  if (B < 0 || n_pos < 1 || n_pos > kMaxCountPositions) return SV_ERR_INVALID_ARG;
  if (!counts || (B > 0 && (!gamma || !accepted))) return SV_ERR_INVALID_ARG;
  if (B == 0) return SV_OK;
  (void)hipGetLastError();
  const hipError_t e = launch_position_counts(B, n_pos, gamma, accepted,
                                              reinterpret_cast<unsigned long long *>(counts),
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

extern "C" sv_status sv_set_gemm_tuning(const char *spec) {
  Tune r;
  if (!parse_tune(spec, r)) return SV_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tune = r;
  return SV_OK;
}
