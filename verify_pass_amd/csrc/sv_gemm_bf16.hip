// GEMM instantiations for bf16 weights.
#include "sv_gemm_kernel.h"

namespace sv {
hipError_t launch_gemm_bf16(const GemmParams &p, int tok_tiles, int depth, int kw, hipStream_t s,
                          int trace_class) {
  return launch_wt<WT_BF16>(p, tok_tiles, depth, kw, s, trace_class);
}
hipError_t launch_gemm_tiled_bf16(const GemmParams &p, hipStream_t s, int trace_class) {
  return launch_tiled(p, s, trace_class);
}
hipError_t launch_gemm_square_bf16(const GemmParams &p, hipStream_t s, int trace_class) {
  return launch_sq(p, s, trace_class);
}
hipError_t launch_gemm_wide_bf16(const GemmParams &p, int tok_tiles, int depth, hipStream_t s, int trace_class) {
  return launch_wide(p, tok_tiles, depth, s, trace_class);
}
}  // namespace sv
