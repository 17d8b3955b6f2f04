// Acceptance entry point that allocates nothing: for callers that cannot
// allocate device memory or pass a workspace (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch memory that sv_accept_commit takes from its workspace (one
// arrival counter per sequence, the per-chunk results, the greedy spill
// space) lives here in a fixed device array.  Each GPU the library runs on
// holds its own copy until the process ends; its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only
// that address is ever passed to kernels.  Every call on a GPU shares the
// array: calls that overlap in time on one GPU race.  The counters, which must
// start at zero, are cleared by a small kernel on the caller's stream before
// the acceptance kernel runs; the rest is written before it is read.
#include <mutex>

#include "sv_common.h"

namespace sv {

// 4 MiB: room for, e.g., greedy acceptance of 9000 stacked rows over a
// 151936-entry vocabulary, or stochastic acceptance of 4096 sequences.
constexpr size_t kAcceptScratchBytes = SV_ACCEPT_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kAcceptScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

// The current device's address of the scratch array (looked up on the first
// call on that device).
hipError_t scratch_address(unsigned char **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<unsigned char *>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

__global__ __launch_bounds__(256) void zero_counters_kernel(int *c, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) c[i] = 0;
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" sv_status sv_accept_commit_noalloc(int32_t B, int32_t V, int32_t mode,
                                              const int32_t *gamma_host, const int32_t *gamma,
                                              const int32_t *draft, const float *p, const float *q,
                                              const float *u_acc, const float *u_samp, int32_t *kv_len,
                                              int32_t *accepted, int32_t *next_token, int32_t *err_flag,
                                              void *stream) {
  AcceptPlan ap;
  const size_t counter_bytes = ((size_t)B * sizeof(int) + 255) / 256 * 256;
  sv_status st = plan_accept(B, V, mode, gamma_host, ap, counter_bytes);
  if (st != SV_OK) return st;
  st = check_accept_args(B, mode, ap, gamma, draft, p, q, u_acc, u_samp, kv_len, accepted, next_token);
  if (st != SV_OK || B == 0) return st;
  if (ap.bytes > kAcceptScratchBytes) return SV_ERR_TOO_LARGE;
  unsigned char *ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return SV_ERR_HIP;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(zero_counters_kernel, dim3((B + 255) / 256), dim3(256), 0, s, reinterpret_cast<int *>(ws), B);
  if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
  return run_accept(B, V, mode, gamma_host, ap, gamma, draft, p, q, u_acc, u_samp, kv_len, accepted,
                    next_token, err_flag, ws, s);
}
