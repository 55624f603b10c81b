// kv_window_noalloc.hip -- swrt_kv_window_append without a caller-owned
// staging buffer, for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// A multi-token step (S > 1) needs its C + S staging rows per (tensor, b, h)
// slice. Here they live in one file-scope device array, `scratch`, that every
// GPU the library runs on holds for the life of the process. Its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept; the host never passes the array's name to a kernel (on
// the host it is only a stand-in symbol). The step then runs the same kernels
// as swrt_kv_window_append with that memory as its staging buffers.
//
// Every call on a GPU shares that GPU's array: calls that overlap in time on
// one GPU (two streams, two host threads) race on it. Nothing in it needs to
// start at zero: the stage phase writes every staging row the commit reads.
#include <mutex>

#include "swrt_host.hpp"

static_assert(SWRT_NOALLOC_STAGING_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) char scratch[SWRT_NOALLOC_STAGING_BYTES];

namespace swrt {
namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices];

// the device address of the current device's scratch array
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SWRT_E_LAUNCH;
  if (dev >= kMaxDevices) return SWRT_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SWRT_E_LAUNCH;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return SWRT_OK;
}

}  // namespace
}  // namespace swrt

using namespace swrt;

extern "C" int swrt_kv_window_append_noalloc(void *k_cache, void *v_cache, const void *k_new,
                                             const void *v_new, const int64_t *new_strides,
                                             const int32_t *cache_past_lens,
                                             const int32_t *evict_counts, int batch,
                                             int kv_heads, int capacity, int seq_len,
                                             int head_dim, int elem_bits, uint32_t *d_flags,
                                             void *stream) {
  if (batch < 0 || kv_heads < 0 || head_dim < 0 || capacity < 1 || seq_len < 1)
    return SWRT_E_INVALID_ARG;
  if (!valid_elem_bits(elem_bits)) return SWRT_E_INVALID_ARG;
  if (seq_len == 1)  // in place: no staging
    return swrt_kv_window_append(k_cache, v_cache, k_new, v_new, new_strides, nullptr, nullptr,
                                 cache_past_lens, evict_counts, batch, kv_heads, capacity,
                                 seq_len, head_dim, elem_bits, SWRT_PHASE_ALL, d_flags, stream);
  // staging [B, H, C + S, D] for K, then V at the next 256-byte boundary
  int64_t rows = 0, bytes = 0;
  if ((int64_t(head_dim) * elem_bits) % 8) return SWRT_E_UNSUPPORTED;
  if (!mul_ok(int64_t(batch) * kv_heads, int64_t(capacity) + seq_len, &rows) ||
      !mul_ok(rows, int64_t(head_dim) * elem_bits / 8, &bytes))
    return SWRT_E_UNSUPPORTED;
  const int64_t half = (bytes + 255) / 256 * 256;
  if (half > SWRT_NOALLOC_STAGING_BYTES / 2) return SWRT_E_UNSUPPORTED;  // beyond the array
  if (bytes == 0)  // nothing to stage: the call is a no-op, as the allocating one
    return swrt_kv_window_append(k_cache, v_cache, k_new, v_new, new_strides, nullptr, nullptr,
                                 cache_past_lens, evict_counts, batch, kv_heads, capacity,
                                 seq_len, head_dim, elem_bits, SWRT_PHASE_ALL, d_flags, stream);
  void *base = nullptr;
  const int st = scratch_address(&base);
  if (st != SWRT_OK) return st;
  char *ks = static_cast<char *>(base);
  return swrt_kv_window_append(k_cache, v_cache, k_new, v_new, new_strides, ks, ks + half,
                               cache_past_lens, evict_counts, batch, kv_heads, capacity, seq_len,
                               head_dim, elem_bits, SWRT_PHASE_ALL, d_flags, stream);
}
