// Paged decode that allocates nothing: attn_paged_decode_gqa_noalloc
// (include/attn.h).  The partial outputs, log-sum-exps and range metadata
// that attn_paged_decode_gqa keeps in the caller's workspace live here in a
// file-scope device array instead, one copy per GPU, reserved when the code
// object is loaded on that GPU and held until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress (the
// device current at the first call on it) and only that address is handed to
// the kernels.  Nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "attn.h"
#include "kernels.h"

namespace {

static_assert(ATTN_DECODE_SCRATCH_BYTES % 256 == 0, "scratch size");

// The no-allocation decode's partial results (see the header for the limit).
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once known

// Device address of `scratch` on the current device (looked up on the first
// call for that device); ATTN_E_HIP if the runtime cannot give it, and
// ATTN_E_INVALID if `stream` belongs to another device (the address would
// not be valid there).
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_E_HIP;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return ATTN_E_HIP;
    if (sdev != dev) return ATTN_E_INVALID;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return ATTN_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_paged_decode_gqa_noalloc(const void* q, const void* k_cache,
                                             const void* v_cache, const int32_t* page_table,
                                             const int32_t* seq_lens, void* o, int B, int H,
                                             int H_kv, int D, int page_size, int num_pages,
                                             int max_pages_per_seq, int dtype, float scale,
                                             hipStream_t stream) {
  // Every argument check first, before any HIP call.
  size_t need = 0;
  const int st = mi355_attn::check_paged_decode(q, k_cache, v_cache, page_table, seq_lens, o, B,
                                                H, H_kv, D, page_size, num_pages,
                                                max_pages_per_seq, dtype, scale, &need);
  if (st != ATTN_OK || need == 0) return st;
  if (need > ATTN_DECODE_SCRATCH_BYTES) return ATTN_E_WORKSPACE;
  void* ws = nullptr;
  const int sa = scratch_address(stream, &ws);
  if (sa != ATTN_OK) return sa;
  // The kernels of the workspace form, with the array as the workspace: they
  // write every partial and the metadata they later read, so nothing needs
  // clearing between calls.
  return attn_paged_decode_gqa(q, k_cache, v_cache, page_table, seq_lens, o, B, H, H_kv, D,
                               page_size, num_pages, max_pages_per_seq, dtype, scale, ws,
                               ATTN_DECODE_SCRATCH_BYTES, stream);
}
