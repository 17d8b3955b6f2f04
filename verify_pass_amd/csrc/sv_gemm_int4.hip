// GEMM instantiations for int4 weights.
#include "sv_gemm_kernel.h"

namespace sv {
hipError_t launch_gemm_int4(const GemmParams &p, int tok_tiles, int depth, int kw, hipStream_t s,
                          int trace_class) {
  return launch_wt<WT_INT4>(p, tok_tiles, depth, kw, s, trace_class);
}
hipError_t launch_gemm_square_int4(const GemmParams &p, hipStream_t s, int trace_class) {
  return launch_sq4(p, s, trace_class);
}
hipError_t launch_gemm_wide_int4(const GemmParams &p, int tok_tiles, hipStream_t s, int trace_class) {
  return launch_wide4(p, tok_tiles, s, trace_class);
}
}  // namespace sv
