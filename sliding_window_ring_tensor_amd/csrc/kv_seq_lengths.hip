// kv_seq_lengths.hip -- lengths of one windowed GQA step, on the device.
//
// onnxruntime pull request "GQA support sliding_window_cache", section
// "Design": the step derives, from seqlens_k alone and on the device (so the
// launches stay graph-capturable), the absolute lengths used for rotary
// positions, the cache-relative lengths used for cache addressing and the
// per-batch eviction count. The follow-up commit of the same pull request does
// this arithmetic in 64 bits (seqlens_k + 1 overflows 32 bits at INT32_MAX)
// and clamps the derived past length at zero; the cache-relative results are
// bounded by the capacity and fit 32 bits again.
//
// One lane per batch entry; the values are independent per entry. With the
// optional work prefix (the exclusive prefix over the batch of the rows each
// entry's step writes, so that one flat grid can map its tiles to (entry,
// row) without a host round trip) one workgroup walks the batch in chunks,
// scanning each chunk within its waves by lane shuffles and across them
// through LDS.
#include "window_device.hpp"

#include "swrt_host.hpp"

namespace swrt {
namespace {

struct LengthArgs {
  const int32_t *seqlens_k;
  int64_t *total, *past;  // may be null
  int32_t *cache_past, *cache_total, *evict;  // cache_total may be null
  uint32_t *flags;
  int32_t batch, S, C;
  FastDiv gap;  // capacity - window + 1
};

__global__ __launch_bounds__(kBlock) void seq_lengths_kernel(LengthArgs a) {
  const int32_t b = blockIdx.x * kBlock + threadIdx.x;
  if (b >= a.batch) return;
  const StepLengths r = step_lengths(a.seqlens_k[b], a.S, a.C, a.gap);
  if (r.bad && a.flags) atomicOr(a.flags, SWRT_FLAG_BAD_SEQLEN);
  if (a.total) a.total[b] = r.T;
  if (a.past) a.past[b] = r.P;
  a.cache_past[b] = int32_t(r.Lp);
  a.evict[b] = int32_t(r.E);
  if (a.cache_total) a.cache_total[b] = int32_t(r.L);
}

// Rows one entry's step writes: S = 1 shifts Lp - E rows when it evicts and
// appends one; S > 1 stages Lp + S rows.
__device__ __forceinline__ int64_t work_rows(const StepLengths &r, int32_t S) {
  return S == 1 ? (r.E > 0 ? r.Lp - r.E : 0) + 1 : r.Lp + S;
}

constexpr int kScanBlock = 1024;  // 16 waves

__global__ __launch_bounds__(kScanBlock) void seq_lengths_scan_kernel(LengthArgs a,
                                                                      int64_t *work) {
  __shared__ int64_t wave_sum[kScanBlock / 64];
  const uint32_t lane = threadIdx.x % 64, wv = threadIdx.x / 64;
  if (threadIdx.x == 0) work[0] = 0;
  int64_t carry = 0;  // rows of the chunks before this one
  for (int32_t base = 0; base < a.batch; base += kScanBlock) {
    const int32_t b = base + int32_t(threadIdx.x);
    int64_t x = 0;
    if (b < a.batch) {
      const StepLengths r = step_lengths(a.seqlens_k[b], a.S, a.C, a.gap);
      if (r.bad && a.flags) atomicOr(a.flags, SWRT_FLAG_BAD_SEQLEN);
      if (a.total) a.total[b] = r.T;
      if (a.past) a.past[b] = r.P;
      a.cache_past[b] = int32_t(r.Lp);
      a.evict[b] = int32_t(r.E);
      if (a.cache_total) a.cache_total[b] = int32_t(r.L);
      x = work_rows(r, a.S);
    }
    // inclusive scan of the wave's 64 values
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t y = __shfl_up(x, d, 64);
      if (lane >= uint32_t(d)) x += y;
    }
    if (lane == 63) wave_sum[wv] = x;
    __syncthreads();
    int64_t before = carry, chunk = 0;
#pragma unroll
    for (int w = 0; w < kScanBlock / 64; ++w) {
      before += uint32_t(w) < wv ? wave_sum[w] : 0;
      chunk += wave_sum[w];
    }
    if (b < a.batch) work[b + 1] = before + x;
    carry += chunk;
    __syncthreads();  // the next chunk rewrites wave_sum
  }
}

}  // namespace
}  // namespace swrt

using namespace swrt;

namespace {

int seq_lengths(const int32_t *seqlens_k, int batch, int seq_len, int capacity, int window,
                int64_t *total_lens, int64_t *past_lens, int32_t *cache_past_lens,
                int32_t *cache_total_lens, int32_t *evict_counts, int64_t *work_offsets,
                uint32_t *d_flags, void *stream) {
  if (batch < 0 || seq_len < 1 || capacity < 1) return SWRT_E_INVALID_ARG;
  if (window < 1 || window > capacity) return SWRT_E_INVALID_ARG;
  const auto addr = [](const void *p) { return uint64_t(reinterpret_cast<uintptr_t>(p)); };
  if (addr(work_offsets) % 8) return SWRT_E_INVALID_ARG;
  if (batch == 0) {  // the prefix of an empty batch is its single 0 (a kernel, not a memset:
    if (!work_offsets) return SWRT_OK;  // the call may be captured into a graph)
    LengthArgs a{};
    hipLaunchKernelGGL(seq_lengths_scan_kernel, dim3(1), dim3(kScanBlock), 0,
                       static_cast<hipStream_t>(stream), a, work_offsets);
    return launch_status();
  }
  if (!seqlens_k || !cache_past_lens || !evict_counts) return SWRT_E_INVALID_ARG;
  if (addr(seqlens_k) % 4 || addr(cache_past_lens) % 4 || addr(evict_counts) % 4 ||
      addr(cache_total_lens) % 4 || addr(total_lens) % 8 || addr(past_lens) % 8 ||
      addr(d_flags) % 4)
    return SWRT_E_INVALID_ARG;
  const uint64_t n4 = uint64_t(batch) * 4, n8 = uint64_t(batch) * 8;
  Range ranges[8] = {range(seqlens_k, n4, false),      range(total_lens, n8, true),
                     range(past_lens, n8, true),        range(cache_past_lens, n4, true),
                     range(cache_total_lens, n4, true), range(evict_counts, n4, true),
                     range(d_flags, 4, true),           range(work_offsets, n8 + 8, true)};
  if (written_overlap(ranges, 8)) return SWRT_E_INVALID_ARG;

  LengthArgs a{seqlens_k, total_lens, past_lens, cache_past_lens, cache_total_lens, evict_counts,
               d_flags, batch, seq_len, capacity, FastDiv(uint32_t(capacity - window + 1))};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (work_offsets) {
    hipLaunchKernelGGL(seq_lengths_scan_kernel, dim3(1), dim3(kScanBlock), 0, s, a, work_offsets);
    return launch_status();
  }
  const uint32_t grid = (uint32_t(batch) + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(seq_lengths_kernel, dim3(grid), dim3(kBlock), 0, s, a);
  return launch_status();
}

}  // namespace

extern "C" int swrt_kv_seq_lengths(const int32_t *seqlens_k, int batch, int seq_len, int capacity,
                                   int64_t *total_lens, int64_t *past_lens,
                                   int32_t *cache_past_lens, int32_t *cache_total_lens,
                                   int32_t *evict_counts, int64_t *work_offsets,
                                   uint32_t *d_flags, void *stream) {
  return seq_lengths(seqlens_k, batch, seq_len, capacity, capacity, total_lens, past_lens,
                     cache_past_lens, cache_total_lens, evict_counts, work_offsets, d_flags,
                     stream);
}

extern "C" int swrt_kv_seq_lengths_drift(const int32_t *seqlens_k, int batch, int seq_len,
                                         int capacity, int window, int64_t *total_lens,
                                         int64_t *past_lens, int32_t *cache_past_lens,
                                         int32_t *cache_total_lens, int32_t *evict_counts,
                                         int64_t *work_offsets, uint32_t *d_flags,
                                         void *stream) {
  return seq_lengths(seqlens_k, batch, seq_len, capacity, window, total_lens, past_lens,
                     cache_past_lens, cache_total_lens, evict_counts, work_offsets, d_flags,
                     stream);
}
