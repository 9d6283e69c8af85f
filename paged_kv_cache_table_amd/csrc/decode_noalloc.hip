// Decode for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// same call as pkv_paged_attn_decode, with its workspace taken from a
// file-scope device array instead of the caller.
//
// Each GPU the library runs on holds its own copy of `scratch`, at its own
// address, until the process ends.  In host code the array's name is only a
// host-side stand-in, so its device address is looked up once per device
// with hipGetSymbolAddress and only that address is ever passed on.
#include <atomic>
#include <cstdio>

#include "pkv_internal.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
// Device address of `scratch` per device (null until the first call on that
// device).  The lookup gives the same address whichever thread makes it, so
// two first calls racing on one device store the same value.
std::atomic<void*> g_scratch_addr[kMaxDevices];

}  // namespace

namespace pkv_host {
void set_error(const char* msg);
}

extern "C" pkv_status pkv_paged_attn_decode_noalloc(const pkv_shape* shape, const void* q,
                                                    const void* k_pool, const void* v_pool,
                                                    const int32_t* block_table, const int32_t* seq_lens,
                                                    int32_t mode, int32_t n_runs, const int32_t* window,
                                                    float* out, float* lse, void* stream) {
  const size_t need = pkv_decode_workspace_bytes(shape, mode, n_runs);
  if (need == 0) {
    // the shape is refused: let the workspace call say why
    return pkv_paged_attn_decode(shape, q, k_pool, v_pool, block_table, seq_lens, mode, n_runs, window, out,
                                 lse, nullptr, 0, stream);
  }
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "this decode needs %zu bytes of workspace, more than the %zu bytes of the built-in scratch; "
             "use pkv_paged_attn_decode with a workspace",
             need, (size_t)PKV_NOALLOC_SCRATCH_BYTES);
    pkv_host::set_error(msg);
    return PKV_E_WORKSPACE;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    char msg[256];
    snprintf(msg, sizeof msg, "no usable current device for the built-in scratch (%s, device %d)",
             hipGetErrorString(e), dev);
    pkv_host::set_error(msg);
    return PKV_E_DEVICE;
  }
  void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      char msg[256];
      snprintf(msg, sizeof msg, "looking up the built-in scratch on device %d: %s", dev, hipGetErrorString(e));
      pkv_host::set_error(msg);
      return PKV_E_DEVICE;
    }
    g_scratch_addr[dev].store(ptr, std::memory_order_release);
  }
  return pkv_paged_attn_decode(shape, q, k_pool, v_pool, block_table, seq_lens, mode, n_runs, window, out, lse,
                               ptr, (size_t)PKV_NOALLOC_SCRATCH_BYTES, stream);
}
