// attn_decode_splitkv_noalloc: the split-KV decode with its workspace in a
// static device array of the library instead of a caller's buffer, for
// callers that cannot allocate device memory.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "attn_decode.h"

namespace lcdg {
attn_status api_fail(attn_status st, const char *msg);
attn_status api_fail_hip(hipError_t e, const char *where);
attn_status decode_run(const attn_decode_args *a, void *workspace, size_t workspace_bytes, attn_stream_t stream,
                       void *const *events);
}  // namespace lcdg

namespace {

constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;

// Partials and arrival counters of attn_decode_splitkv_noalloc; every GPU the
// library runs on holds its own copy until the process ends.  In host code
// this name stands for no device address: host code uses only the address
// hipGetSymbolAddress returns for the current device (g_scratch).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch[kMaxDevices] = {nullptr};

// The current device's copy of the scratch array, looked up on the first
// call on that device (with it current) and kept.
attn_status scratch_on_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return lcdg::api_fail_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return lcdg::api_fail(ATTN_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return lcdg::api_fail_hip(e, "hipGetSymbolAddress(scratch)");
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255))
      return lcdg::api_fail(ATTN_ERR_HIP, "static scratch is not a 256-byte aligned device address");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" attn_status attn_decode_splitkv_noalloc(const attn_decode_args *a, attn_stream_t stream) {
  if (!a) return lcdg::api_fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->workspace || a->workspace_bytes)
    return lcdg::api_fail(ATTN_ERR_INVALID_ARG,
                          "attn_decode_splitkv_noalloc uses the library's static scratch: workspace must be NULL "
                          "and workspace_bytes 0");
  size_t need = 0;
  attn_status st = attn_decode_workspace_size(a, &need);
  if (st != ATTN_OK) return st;
  if (need > kScratchBytes) {
    const std::string msg = "attn_decode_splitkv_noalloc: these arguments need " + std::to_string(need) +
                            " bytes of scratch, above the static scratch of " + std::to_string(kScratchBytes) +
                            " bytes (use attn_decode_splitkv with a workspace)";
    return lcdg::api_fail(ATTN_ERR_WORKSPACE_TOO_SMALL, msg.c_str());
  }
  if (a->kv.B == 0) return ATTN_OK;
  void *ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != ATTN_OK) return st;
  return lcdg::decode_run(a, ws, kScratchBytes, stream, nullptr);
}
