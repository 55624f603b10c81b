// swrt_host.hpp -- host-side validation ("plans") shared by the entry points.
//
// A plan checks every argument of a call, gathers the byte ranges the call
// touches (for the overlap check) and the OR of every address, stride and row
// size (for the copy word), and holds the launch geometry once the word is
// chosen. Nothing here touches the device.
#pragma once

#include "scatter_device.hpp"
#include "window_device.hpp"

namespace swrt {

constexpr int kMaxLayers = SWRT_MAX_LAYERS;    // layers per batched window launch
constexpr int kMaxTensors = SWRT_MAX_BATCHED;  // tensors per batched scatter launch

// widest word (16, 8, 4, 2, 1 bytes) dividing every value OR-ed into `acc`
inline int word_of(uint64_t acc) {
  return acc % 16 == 0 ? 16 : acc % 8 == 0 ? 8 : acc % 4 == 0 ? 4 : acc % 2 == 0 ? 2 : 1;
}

inline uint64_t addr_of(const void *p) { return uint64_t(reinterpret_cast<uintptr_t>(p)); }

// element alignment a pointer must have: the element size, capped at 8 bytes
// (complex128 is two doubles)
inline uint64_t elem_align(int elem_bits) {
  return elem_bits >= 16 ? uint64_t(elem_bits / 8 > 8 ? 8 : elem_bits / 8) : 1;
}

struct WindowPlan {
  WindowGeom g;
  char *cache[kMaxLayers][2];
  const char *nw[kMaxLayers][2];
  char *stage[kMaxLayers][2];
  int n_layers;
  uint32_t slices;
  uint64_t align;  // OR of addresses, strides and the row size
  int64_t row;     // row bytes
  bool empty;      // nothing to launch
};

// Validate a windowed step. With lengths_in_kernel, cache_past_lens and
// evict_counts are not used (the kernel derives them from seqlens_k).
int plan_window(int n_layers, void *const *k_caches, void *const *v_caches,
                const void *const *k_news, const void *const *v_news, const int64_t *new_strides,
                void *const *k_stagings, void *const *v_stagings, const int32_t *cache_past_lens,
                const int32_t *evict_counts, bool lengths_in_kernel, int batch, int kv_heads,
                int capacity, int seq_len, int head_dim, int elem_bits, unsigned phase,
                uint32_t *d_flags, WindowPlan *p, Range *ranges, int *nr);

// Fill the word-dependent geometry; SWRT_E_UNSUPPORTED past the size limits.
int finish_window(WindowPlan *p, int vec);

struct ScatterPlan {
  ScatterGeom g;
  char *present[kMaxTensors];
  const char *past[kMaxTensors];
  const char *update[kMaxTensors];
  int n;
  bool in_place;
  bool empty;      // nothing to launch
  uint64_t align;  // OR of addresses and the row size
  int64_t row;     // row bytes
  int64_t rows;    // rows per tensor the kernel walks (update rows in place, present rows otherwise)
  int64_t O, B;
  uint32_t tiles;  // tiles per tensor
};

int plan_scatter(int n_tensors, void *const *presents, const void *const *pasts,
                 const void *const *updates, const int64_t *write_indices, const int64_t *shape,
                 int rank, int axis, int64_t seq_len, int mode, int elem_bits, uint32_t *d_flags,
                 ScatterPlan *p, Range *ranges, int *nr);

// tile_words: words per workgroup tile of the kernel that will run the plan
int finish_scatter(ScatterPlan *p, int vec, uint32_t tile_words);

}  // namespace swrt
