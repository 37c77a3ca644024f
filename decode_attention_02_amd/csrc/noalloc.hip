// gqla_decode_absorb_noalloc: gqla_decode_absorb for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). The split-KV partial results live in a fixed array in the library's own
// device memory instead of a caller workspace; everything else is gqla_decode_absorb.
#include "../../include/gqla.h"
#include "gqla_internal.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

namespace {

constexpr size_t kScratchBytes = GQLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// One copy per GPU, held from the library's load until the process ends. Host code never
// uses this name as an address: the per-device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once known

gqla_status error(gqla_status s, const char* msg) {
  gqla::set_last_error(msg);
  return s;
}

// Address of the scratch array on the calling thread's current device (looked up once per
// device, with that device current).
gqla_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return error(GQLA_ERR_HIP, "gqla_decode_absorb_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return error(GQLA_ERR_UNSUPPORTED, "gqla_decode_absorb_noalloc: device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      char msg[256];
      snprintf(msg, sizeof msg, "gqla_decode_absorb_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
               hipGetErrorString(e));
      return error(GQLA_ERR_HIP, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return GQLA_OK;
}

}  // namespace

extern "C" gqla_status gqla_decode_absorb_noalloc(const gqla_dims* dims, const gqla_paged* paged,
                                                  const void* q_abs, const void* latent_cache, float* o_lat,
                                                  float* lse, void* stream) {
  size_t need = 0;
  gqla_status st = gqla_workspace_bytes(dims, paged, GQLA_PATH_ABSORB, &need);
  if (st != GQLA_OK) return st;
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "gqla_decode_absorb_noalloc: the split-KV plan needs %zu bytes of scratch, more than the %zu the "
             "library holds; use gqla_decode_absorb with a workspace",
             need, kScratchBytes);
    return error(GQLA_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  if (need > 0 && (st = scratch_of_current_device(&ws)) != GQLA_OK) return st;
  return gqla_decode_absorb(dims, paged, q_abs, latent_cache, ws, need > 0 ? kScratchBytes : 0, o_lat, lse, stream);
}
