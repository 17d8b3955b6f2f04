// Weight-streaming GEMM over the stacked verify tokens, gfx950.
//
// Y^T[N][T] = W[N][K] * X^T: weight rows are the MFMA's M side and tokens its
// N side.  One read of the weights serves every stacked token of every
// sequence -- the single weight stream a verification pass is built around.
//
// Work unit: 32 weight rows (two 16-row MFMA tiles) x up to 64 tokens x one
// split of K, run by KW waves of one workgroup that each take a consecutive
// piece of the split.  A wave streams its weight rows straight from HBM into
// registers with a grouped prefetch and reads the (small, L2-resident) token
// rows directly as MFMA B operands: no LDS staging in the main loop.  With
// KW > 1 the pieces are added through LDS in wave order at the end.
//
// The two tiles of a unit are chosen so that every epilogue is lane-local:
//   QKV     tile 0 = rotation-pair firsts, tile 1 = their partners (i + hd/2):
//           RMSNorm scale, RoPE, q to a staging buffer, k/v appended to caches
//   SWIGLU  tile 0 = gate rows, tile 1 = the matching up rows: silu(g) * u
//   RESID   + residual (O and down projections)
//   LOGITS  fp32 logits and per-(32 rows, token) softmax statistics
// RMSNorm only needs a per-token scale r_t = 1/sqrt(mean(x^2) + eps):
// (r_t x) W = r_t (x W), so it is applied in the epilogue from sums of squares
// of the token operand the unit already loads.
//
// K splits across units: for the remaining cases with too few row groups to
// occupy the chip, units also split K.  Each split stores its fp32 partial tile with device-scope (sc1)
// stores, waits for them to complete and bumps a per-tile counter; the split
// that arrives last reads the partials back with device-scope loads, adds
// them in split order (bitwise repeatable) and runs the epilogue.  No
// cache-wide fence is involved.
#include "sv_common.h"

namespace sv {

hipError_t launch_gemm_bf16(const GemmParams &p, int tok_tiles, int depth, int kw, hipStream_t s,
                          int trace_class);
hipError_t launch_gemm_int4(const GemmParams &p, int tok_tiles, int depth, int kw, hipStream_t s,
                          int trace_class);
hipError_t launch_gemm_f32(const GemmParams &p, int tok_tiles, int depth, int kw, hipStream_t s,
                         int trace_class);

hipError_t launch_gemm_tiled_bf16(const GemmParams &p, hipStream_t s, int trace_class);
hipError_t launch_gemm_square_bf16(const GemmParams &p, hipStream_t s, int trace_class);
hipError_t launch_gemm_square_int4(const GemmParams &p, hipStream_t s, int trace_class);
hipError_t launch_gemm_wide_bf16(const GemmParams &p, int tok_tiles, int depth, hipStream_t s, int trace_class);
hipError_t launch_gemm_wide_int4(const GemmParams &p, int tok_tiles, hipStream_t s, int trace_class);

hipError_t launch_gemm(const GemmParams &p, int wtype, int tok_tiles, int depth, int kw, hipStream_t s,
                       int trace_class) {
  if (kw == kGemmTiled) {
    if (wtype != WT_BF16 || !p.packed || p.splits != 1) return hipErrorInvalidValue;
    return launch_gemm_tiled_bf16(p, s, trace_class);
  }
  if (kw == kGemmSquare) {
    if ((wtype != WT_BF16 && wtype != WT_INT4) || !p.packed) return hipErrorInvalidValue;
    // K splits: at least one half step (of 32) each; partial tiles per 128 tokens
    if (p.splits < 1 || p.splits > 2 * p.ksteps || (p.splits > 1 && p.ntblk != (p.T + 127) / 128))
      return hipErrorInvalidValue;
    return wtype == WT_INT4 ? launch_gemm_square_int4(p, s, trace_class) : launch_gemm_square_bf16(p, s, trace_class);
  }
  if (kw == kGemmWide) {
    if (!p.packed) return hipErrorInvalidValue;
    if (wtype == WT_INT4) {
      if (tok_tiles != 1 && tok_tiles != 2 && tok_tiles != 4 && tok_tiles != 8) return hipErrorInvalidValue;
      return launch_gemm_wide_int4(p, tok_tiles, s, trace_class);
    }
    if (tok_tiles != 4 && tok_tiles != 8) return hipErrorInvalidValue;
    if (wtype != WT_BF16) return hipErrorInvalidValue;
    return launch_gemm_wide_bf16(p, tok_tiles, depth, s, trace_class);
  }
  if (wtype == WT_BF16) return launch_gemm_bf16(p, tok_tiles, depth, kw, s, trace_class);
  if (wtype == WT_INT4) return launch_gemm_int4(p, tok_tiles, depth, kw, s, trace_class);
  return launch_gemm_f32(p, tok_tiles, depth, kw, s, trace_class);
}

namespace {
// One thread per 16-byte fragment of the packed layout (see sv_pack_matrix).
// Packed layout: step-major -- K step s of every 32-row group g in turn,
// each holding the group's two 16-row tiles a back to back, each tile as
// lane-ordered 16-byte MFMA fragments.  One thread per 16-byte fragment.
__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint16_t *src, uint4 *dst, int N, int K) {
  const int ks = K / 64;
  const size_t ng = (size_t)(N + 31) / 32;
  const size_t total = ng * ks * 256;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  // idx = (((step * ng + g) * 2 + a) * 2 + m) * 64 + lane
  const int lane = idx & 63, m = (idx >> 6) & 1, a = (idx >> 7) & 1;
  const size_t sg = idx >> 8;
  const size_t g = sg % ng;
  const int step = (int)(sg / ng);
  const size_t row = g * 32 + a * 16 + (lane & 15);
  const int k = step * 64 + 32 * m + 8 * (lane >> 4);
  dst[idx] = row < (size_t)N ? *reinterpret_cast<const uint4 *>(src + row * K + k) : uint4{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(256) void pack_int4_kernel(const uint32_t *src, const uint16_t *ssrc, uint4 *dst,
                                                        uint16_t *sdst, int N, int K) {
  const int ks = K / 128;
  const size_t ng = (size_t)(N + 31) / 32;
  const size_t total = ng * ks * 128;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  // idx = ((step * ng + g) * 2 + a) * 64 + lane
  const int lane = idx & 63, a = (idx >> 6) & 1;
  const size_t sg = idx >> 7;
  const size_t g = sg % ng;
  const int step = (int)(sg / ng);
  const size_t row = g * 32 + a * 16 + (lane & 15);
  const int gq = lane >> 4;
  if (row < (size_t)N) {
    dst[idx] = *reinterpret_cast<const uint4 *>(src + row * (K / 8) + step * 16 + 4 * gq);
    sdst[idx] = ssrc[row * (K / 32) + step * 4 + gq];
  } else {
    dst[idx] = uint4{0u, 0u, 0u, 0u};
    sdst[idx] = 0;
  }
}

}  // namespace

hipError_t launch_pack(int wtype, int N, int K, const void *w, const void *scale, void *wp, void *sp,
                       hipStream_t s) {
  const size_t groups = (size_t)(N + 31) / 32;
  if (wtype == WT_BF16) {
    const size_t total = groups * (K / 64) * 256;
    hipLaunchKernelGGL(pack_bf16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint16_t *>(w), static_cast<uint4 *>(wp), N, K);
  } else {
    const size_t total = groups * (K / 128) * 128;
    hipLaunchKernelGGL(pack_int4_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint32_t *>(w), static_cast<const uint16_t *>(scale),
                       static_cast<uint4 *>(wp), static_cast<uint16_t *>(sp), N, K);
  }
  return hipGetLastError();
}

size_t gemm_partial_floats(int ngroups, int splits, int ntblk, int tok_tiles) {
  if (splits <= 1) return 0;
  return (size_t)splits * ngroups * ntblk * (2 * tok_tiles * 4 * 64);
}

}  // namespace sv
