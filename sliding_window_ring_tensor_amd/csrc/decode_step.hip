// decode_step.hip -- every KV-cache update of one decode step in one launch.
//
// A model whose layers use windowed caches (onnxruntime pull request "GQA
// support sliding_window_cache", section "Design") and full max-length caches
// updated by TensorScatter in linear mode (ONNX operator page "TensorScatter")
// gets one new K and V row per (batch, kv-head) and layer at every decode
// step. swrt_kv_decode_step does, in one grid, exactly what these three calls
// do in three launches:
//
//   swrt_kv_seq_lengths(seqlens_k, B, 1, C, T, P, Lp, L, E)
//   swrt_kv_window_append_layers(all windowed layers, Lp, E, S = 1)
//   swrt_tensor_scatter_batched(all full caches in place, write_indices,
//                               [B, H, M, D], axis 2, S = 1, linear)
//
// Workgroup roles (uniform per workgroup): the first workgroups carry the
// full-cache row writes, the rest one windowed slice each; every window
// workgroup derives its own (Lp, E) from seqlens_k with the same arithmetic
// as kv_seq_lengths (or kv_seq_lengths_drift when window < capacity), and the
// first workgroups (one batch entry per lane) also write the
// length arrays for the attention that follows. Two kernel boundaries per
// step disappear, and with them their dispatch and cache-maintenance cost.
// The XF instances (swrt_kv_decode_step_xf) fuse the row transform of
// xf_device.hpp into every write: windowed rows at position P = T - 1, full
// caches at their write index; full caches alternate K and V.
#include "swrt_host.hpp"

namespace swrt {
namespace {

struct DecodeArgs {
  char *wc[kMaxLayers][2];        // windowed caches
  const char *wn[kMaxLayers][2];  // windowed new rows
  char *fc[kMaxTensors];          // full caches
  const char *fu[kMaxTensors];    // full-cache new rows
  WindowGeom wg;
  ScatterGeom sg;
  const int32_t *seqlens_k;
  int64_t *total, *past;
  int32_t *cache_past, *cache_total, *evict;
  uint32_t full_tiles, full_blocks, win_blocks, len_blocks;
  int32_t batch;
  FastDiv gap;  // capacity - window + 1
  RowXf xf;     // fused append only
};

// BLOCK x UNROLL: the window shape (512 x 2 for the base layout; one wave,
// 64 x 16, for the drifting layout, whose steps are mostly single-row appends).
// DRIFT: window < capacity (the lengths take the gap). XF: fused append.
template <int VEC, int SPW, int BLOCK, int UNROLL, bool DRIFT, bool XF>
__global__ __launch_bounds__(BLOCK) void decode_step_kernel(DecodeArgs a) {
  constexpr uint32_t kFullTile = BLOCK * kScatUnroll;  // full-cache words per workgroup
  __shared__ TileBatches<kFullTile, XF> tb;
  const uint32_t bid = blockIdx.x;
  if (bid < a.len_blocks) {  // the length arrays (no barrier in this part)
    const int32_t b = int32_t(bid * BLOCK + threadIdx.x);
    if (b < a.batch) {
      const StepLengths r = step_lengths<DRIFT>(a.seqlens_k[b], 1, a.wg.C, a.gap);
      if (r.bad && a.wg.flags) atomicOr(a.wg.flags, SWRT_FLAG_BAD_SEQLEN);
      if (a.total) a.total[b] = r.T;
      if (a.past) a.past[b] = r.P;
      if (a.cache_past) a.cache_past[b] = int32_t(r.Lp);
      if (a.cache_total) a.cache_total[b] = int32_t(r.L);
      if (a.evict) a.evict[b] = int32_t(r.E);
    }
  }
  if (bid < a.full_blocks) {  // full caches: TensorScatter rows in place
    const uint32_t t = bid / a.full_tiles;
    // fused append: 4-byte words at most, so each lane transforms few elements
    constexpr int VS = XF && VEC > 4 ? 4 : VEC;
    scatter_in_place_tile<VS, BLOCK, XF>(a.sg, a.fc[t], a.fu[t],
                                         (bid - t * a.full_tiles) * kFullTile, tb, &a.xf,
                                         int(t & 1));
    return;
  }
  const uint32_t wb = bid - a.full_blocks;
  if (wb >= a.win_blocks) return;  // a grid sized by the length arrays alone
  // the window workgroup's slice(s); (Lp, E) from seqlens_k, always a valid pair
  const auto work = [&](uint32_t slice, int g) {
    const Slice s = decode_slice(a.wg, slice);
    // a group kernel's wave reads its own slice's entry by a scalar load
    // (the fp8 step: 33.5 -> 32.7 us); the one-slice workgroups keep the
    // vector load, which measured 0.5 us faster on the bf16 step
    const int32_t sk = SPW > 1 ? ld_invariant(a.seqlens_k, s.b) : a.seqlens_k[s.b];
    const StepLengths r = step_lengths<DRIFT>(sk, 1, a.wg.C, a.gap);
    SliceWork w;
    w.Lp = r.Lp;
    w.E = r.E;
    w.t = int(s.t);
    w.h = s.h;
    w.pos = r.P;
    w.ok = true;
    if constexpr (XF) w.ok = positions_ok(a.wg, a.xf, s, threadIdx.x == g * (BLOCK / SPW), r.P);
    w.base = a.wc[s.layer][s.t] + uint64_t(s.b * a.wg.H + s.h) * uint64_t(a.wg.C) * a.wg.row_bytes;
    w.new_row = a.wn[s.layer][s.t] + s.b * a.wg.nb_b + s.h * a.wg.nb_h;
    return w;
  };
  if constexpr (SPW == 1) {
    const SliceWork w = work(wb, 0);
    if (!w.ok) return;
    shift_append_slice<VEC, BLOCK, UNROLL, XF>(w.base, w.new_row, w.Lp, w.E, a.wg.row_bytes,
                                               a.wg.row_words, &a.xf, w.t, w.pos, w.h);
  } else {
    shift_append_group<VEC, SPW, XF>(wb * SPW, a.wg.slices, a.wg.row_bytes, a.wg.row_words, work,
                                     &a.xf);
  }
}

template <int VEC, bool XF>
void launch_decode(const DecodeArgs &a, bool drift, int spw, uint64_t grid, hipStream_t s) {
  if (drift)
    hipLaunchKernelGGL((decode_step_kernel<VEC, 1, kWaveBlock, kWaveUnroll, true, XF>),
                       dim3(grid), dim3(kWaveBlock), 0, s, a);
  else if (spw == 4)
    hipLaunchKernelGGL((decode_step_kernel<VEC, 4, kWinBlock, kWinUnroll, false, XF>),
                       dim3(grid), dim3(kWinBlock), 0, s, a);
  else if (spw == 2)
    hipLaunchKernelGGL((decode_step_kernel<VEC, 2, kWinBlock, kWinUnroll, false, XF>),
                       dim3(grid), dim3(kWinBlock), 0, s, a);
  else
    hipLaunchKernelGGL((decode_step_kernel<VEC, 1, kWinBlock, kWinUnroll, false, XF>),
                       dim3(grid), dim3(kWinBlock), 0, s, a);
}

template <bool XF>
void launch_vec(int vec, const DecodeArgs &a, bool drift, int spw, uint64_t grid, hipStream_t s) {
  switch (vec) {
    case 16: launch_decode<16, XF>(a, drift, spw, grid, s); break;
    case 8: launch_decode<8, XF>(a, drift, spw, grid, s); break;
    case 4: launch_decode<4, XF>(a, drift, spw, grid, s); break;
    case 2: launch_decode<2, XF>(a, drift, spw, grid, s); break;
    default: launch_decode<1, XF>(a, drift, spw, grid, s); break;
  }
}

}  // namespace
}  // namespace swrt

using namespace swrt;

namespace {

// xf: the fused append (null: plain copies); full caches then alternate K, V
int decode_step(int n_window_layers, void *const *win_k_caches, void *const *win_v_caches,
                const void *const *win_k_new, const void *const *win_v_new,
                const int64_t *win_new_strides, const int32_t *seqlens_k, int capacity, int window,
                int64_t *total_lens, int64_t *past_lens, int32_t *cache_past_lens,
                int32_t *cache_total_lens, int32_t *evict_counts, int n_full,
                void *const *full_caches, const void *const *full_new,
                const int64_t *write_indices, int max_seq, int batch, int kv_heads, int head_dim,
                int elem_bits, const swrt_row_transform *xf, uint32_t *d_flags, void *stream) {
  if (batch < 0 || capacity < 1 || n_window_layers < 0 || n_full < 0) return SWRT_E_INVALID_ARG;
  if (window < 1 || window > capacity) return SWRT_E_INVALID_ARG;
  WindowPlan wp{};
  ScatterPlan sp{};
  Range ranges[6 * kMaxLayers + 3 * kMaxTensors + 24];
  int nr = 0;
  RowXf x{};
  int st;
  if (xf) {
    if ((st = plan_xf(xf, head_dim, kv_heads, &x, ranges, &nr)) != SWRT_OK) return st;
    elem_bits = x.out_bytes * 8;
  }
  st = plan_window(n_window_layers, win_k_caches, win_v_caches, win_k_new, win_v_new,
                   win_new_strides, nullptr, nullptr, nullptr, nullptr, true, batch, kv_heads,
                   capacity, 1, head_dim, elem_bits, SWRT_PHASE_ALL, d_flags, xf ? &x : nullptr,
                   &wp, ranges, &nr);
  if (st != SWRT_OK) return st;
  const int64_t shape[4] = {batch, kv_heads, max_seq, head_dim};
  sp.empty = true;
  if (n_full > 0) {
    st = plan_scatter(n_full, full_caches, const_cast<const void *const *>(full_caches), full_new,
                      write_indices, shape, 4, 2, 1, SWRT_MODE_LINEAR, elem_bits, d_flags,
                      xf ? &x : nullptr, &sp, ranges, &nr);
    if (st != SWRT_OK) return st;
  }
  const bool lengths_out = total_lens || past_lens || cache_past_lens || cache_total_lens ||
                           evict_counts;
  if ((lengths_out || !wp.empty) && batch > 0 && !seqlens_k) return SWRT_E_INVALID_ARG;
  const uint64_t B = uint64_t(batch);
  if (addr_of(seqlens_k) % 4 || addr_of(total_lens) % 8 || addr_of(past_lens) % 8 ||
      addr_of(cache_past_lens) % 4 || addr_of(cache_total_lens) % 4 || addr_of(evict_counts) % 4)
    return SWRT_E_INVALID_ARG;
  ranges[nr++] = range(seqlens_k, B * 4, false);
  ranges[nr++] = range(total_lens, B * 8, true);
  ranges[nr++] = range(past_lens, B * 8, true);
  ranges[nr++] = range(cache_past_lens, B * 4, true);
  ranges[nr++] = range(cache_total_lens, B * 4, true);
  ranges[nr++] = range(evict_counts, B * 4, true);
  ranges[nr++] = range(d_flags, 4, true);
  if (written_overlap(ranges, nr)) return SWRT_E_INVALID_ARG;

  const bool do_len = lengths_out && batch > 0;
  if (wp.empty && sp.empty && !do_len) return SWRT_OK;
  // one copy word for both parts: the rows have the same size
  const int vec = word_of((wp.empty ? 0 : wp.align) | (sp.empty ? 0 : sp.align) |
                          uint64_t(wp.empty && sp.empty ? 16 : 0));
  if (!wp.empty && (st = finish_window(&wp, vec)) != SWRT_OK) return st;
  // the drifting layout runs the one-wave shape (see decode_step_kernel)
  const bool drift = window < capacity;
  const int block = drift ? kWaveBlock : kWinBlock;
  if (xf && head_dim > kXfLaneElems * block) return SWRT_E_UNSUPPORTED;  // XfLanes per lane
  const int vec_s = xf && vec > 4 ? 4 : vec;  // the full caches' word (see decode_step_kernel)
  if (!sp.empty && (st = finish_scatter(&sp, vec_s, uint32_t(block * kScatUnroll))) != SWRT_OK)
    return st;

  static_assert(sizeof(DecodeArgs) <= 4096, "kernel arguments exceed 4 KiB");
  DecodeArgs a;
  for (int l = 0; l < n_window_layers && !wp.empty; ++l)
    for (int t = 0; t < 2; ++t) {
      a.wc[l][t] = wp.cache[l][t];
      a.wn[l][t] = wp.nw[l][t];
    }
  for (int t = 0; t < n_full && !sp.empty; ++t) {
    a.fc[t] = sp.present[t];
    a.fu[t] = sp.update[t];
  }
  a.wg = wp.g;
  a.wg.C = capacity;
  a.wg.flags = d_flags;
  a.sg = sp.g;
  a.seqlens_k = seqlens_k;
  a.total = total_lens;
  a.past = past_lens;
  a.cache_past = cache_past_lens;
  a.cache_total = cache_total_lens;
  a.evict = evict_counts;
  a.batch = batch;
  a.gap = FastDiv(uint32_t(capacity - window + 1));
  a.xf = x;
  a.full_tiles = sp.empty ? 1 : sp.tiles;
  a.full_blocks = sp.empty ? 0 : sp.tiles * uint32_t(sp.n);
  a.len_blocks = do_len ? uint32_t((B + block - 1) / block) : 0;
  const int spw = wp.empty || drift ? 1
                                    : slices_per_group(capacity, wp.g.row_words, xf != nullptr,
                                                       xf ? int64_t(head_dim) : 0);
  a.win_blocks = wp.empty ? 0 : (wp.slices + spw - 1) / spw;
  uint64_t grid = uint64_t(a.full_blocks) + a.win_blocks;
  if (grid < a.len_blocks) grid = a.len_blocks;  // length arrays alone
  if (grid >= (uint64_t(1) << 31)) return SWRT_E_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (xf)
    launch_vec<true>(vec, a, drift, spw, grid, s);
  else
    launch_vec<false>(vec, a, drift, spw, grid, s);
  return launch_status();
}

}  // namespace

extern "C" int swrt_kv_decode_step(int n_window_layers, void *const *win_k_caches,
                                   void *const *win_v_caches, const void *const *win_k_new,
                                   const void *const *win_v_new, const int64_t *win_new_strides,
                                   const int32_t *seqlens_k, int capacity, int window,
                                   int64_t *total_lens, int64_t *past_lens,
                                   int32_t *cache_past_lens, int32_t *cache_total_lens,
                                   int32_t *evict_counts, int n_full, void *const *full_caches,
                                   const void *const *full_new, const int64_t *write_indices,
                                   int max_seq, int batch, int kv_heads, int head_dim,
                                   int elem_bits, uint32_t *d_flags, void *stream) {
  return decode_step(n_window_layers, win_k_caches, win_v_caches, win_k_new, win_v_new,
                     win_new_strides, seqlens_k, capacity, window, total_lens, past_lens,
                     cache_past_lens, cache_total_lens, evict_counts, n_full, full_caches,
                     full_new, write_indices, max_seq, batch, kv_heads, head_dim, elem_bits,
                     nullptr, d_flags, stream);
}

extern "C" int swrt_kv_decode_step_xf(
    int n_window_layers, void *const *win_k_caches, void *const *win_v_caches,
    const void *const *win_k_new, const void *const *win_v_new, const int64_t *win_new_strides,
    const int32_t *seqlens_k, int capacity, int window, int64_t *total_lens, int64_t *past_lens,
    int32_t *cache_past_lens, int32_t *cache_total_lens, int32_t *evict_counts,
    int n_full_layers, void *const *full_k_caches, void *const *full_v_caches,
    const void *const *full_k_new, const void *const *full_v_new, const int64_t *write_indices,
    int max_seq, int batch, int kv_heads, int head_dim, const swrt_row_transform *xf,
    uint32_t *d_flags, void *stream) {
  if (!xf || n_full_layers < 0 || n_full_layers > kMaxTensors / 2) return SWRT_E_INVALID_ARG;
  if (n_full_layers > 0 && (!full_k_caches || !full_v_caches || !full_k_new || !full_v_new))
    return SWRT_E_INVALID_ARG;
  void *caches[kMaxTensors];
  const void *news[kMaxTensors];
  for (int l = 0; l < n_full_layers; ++l) {  // K, V, K, V, ...: tensor = index & 1
    caches[2 * l] = full_k_caches[l];
    caches[2 * l + 1] = full_v_caches[l];
    news[2 * l] = full_k_new[l];
    news[2 * l + 1] = full_v_new[l];
  }
  return decode_step(n_window_layers, win_k_caches, win_v_caches, win_k_new, win_v_new,
                     win_new_strides, seqlens_k, capacity, window, total_lens, past_lens,
                     cache_past_lens, cache_total_lens, evict_counts, 2 * n_full_layers, caches,
                     news, write_indices, max_seq, batch, kv_heads, head_dim, 8, xf, d_flags,
                     stream);
}
