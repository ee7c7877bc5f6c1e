// mm_ssd_forward_noalloc: mm_ssd_forward with its workspace taken from a
// fixed device array compiled into the library, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid allocation).  Declared in include/mm_ssd.h.
//
// The array lives in device memory of every GPU the library runs on, from
// the first call on that GPU until the process ends.  Its address is taken
// once per device with hipGetSymbolAddress (the array's name in host code is
// only a host-side handle, not a device address) and kept per device; the
// kernels receive that pointer exactly as they receive a caller's workspace.
// No call allocates: workspace sizes above the array are rejected before
// anything is enqueued.  Nothing in the scan's workspace needs to start at
// zero: every byte a call reads (tile fragments, head-major dt, segment
// states and decays) is written earlier in the same call.  Calls that overlap
// on one GPU (other streams, or other host threads) share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mm_ssd.h"

namespace {

constexpr size_t kScratchBytes = MM_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size keeps 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device

// Device address of the array on the current device (looked up on the first
// call there, with that device current).
int scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MM_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MM_OK;
}

}  // namespace

extern "C" int mm_ssd_forward_noalloc(const void* x, int64_t x_row_stride, const void* dt,
                                      int64_t dt_row_stride, const float* A, const void* B,
                                      int64_t b_row_stride, const void* C, int64_t c_row_stride,
                                      const float* D, void* y, int64_t y_row_stride,
                                      const float* initial_state, float* final_state,
                                      int64_t batch, int64_t seqlen, int64_t n_heads,
                                      int64_t d_head, int64_t d_state, int64_t ngroups,
                                      int64_t n_heads_active, int64_t chunk, int dtype,
                                      void* stream) {
  size_t need = 0;
  int st = mm_ssd_forward_workspace_size(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                         n_heads_active, chunk, dtype, &need);
  if (st != MM_OK) return st;
  if (need > kScratchBytes) return MM_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_on_current_device(&ws);
    if (st != MM_OK) return st;
  }
  return mm_ssd_forward(x, x_row_stride, dt, dt_row_stride, A, B, b_row_stride, C, c_row_stride,
                        D, y, y_row_stride, initial_state, final_state, batch, seqlen, n_heads,
                        d_head, d_state, ngroups, n_heads_active, chunk, dtype, ws,
                        need > 0 ? kScratchBytes : 0, stream);
}
