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
  RowXf xf;  // the fused append's transform (zero for a plain copy)
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
// evict_counts are not used (the kernel derives them from seqlens_k). With
// xf (a checked transform, see plan_xf), new rows hold xf->in_type elements
// and caches elem_bits = 8 * xf->out_bytes.
int plan_window(int n_layers, void *const *k_caches, void *const *v_caches,
                const void *const *k_news, const void *const *v_news, const int64_t *new_strides,
                void *const *k_stagings, void *const *v_stagings, const int32_t *cache_past_lens,
                const int32_t *evict_counts, bool lengths_in_kernel, int batch, int kv_heads,
                int capacity, int seq_len, int head_dim, int elem_bits, unsigned phase,
                uint32_t *d_flags, const RowXf *xf, WindowPlan *p, Range *ranges, int *nr);

// Fill the word-dependent geometry; SWRT_E_UNSUPPORTED past the size limits.
int finish_window(WindowPlan *p, int vec);

struct ScatterPlan {
  ScatterGeom g;
  RowXf xf;  // the fused append's transform (zero for a plain copy)
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

// With xf, update rows hold xf->in_type elements (axis must be rank - 2) and
// caches elem_bits = 8 * xf->out_bytes.
int plan_scatter(int n_tensors, void *const *presents, const void *const *pasts,
                 const void *const *updates, const int64_t *write_indices, const int64_t *shape,
                 int rank, int axis, int64_t seq_len, int mode, int elem_bits, uint32_t *d_flags,
                 const RowXf *xf, ScatterPlan *p, Range *ranges, int *nr);

// tile_words: words per workgroup tile of the kernel that will run the plan
int finish_scatter(ScatterPlan *p, int vec, uint32_t tile_words);

// Check a row transform for rows of head_dim elements of `heads` KV heads
// and fill the device form; the rotary and per-channel tables join the
// read-only ranges of the call.
inline int plan_xf(const swrt_row_transform *t, int64_t head_dim, int64_t heads, RowXf *x,
                   Range *ranges, int *nr) {
  const auto bytes = [](int type) {
    return type == SWRT_XF_F32 ? 4 : type == SWRT_XF_F16 || type == SWRT_XF_BF16 ? 2
                                 : type == SWRT_XF_INT8 || type == SWRT_XF_UINT8 ||
                                           type == SWRT_XF_FP8_E4M3
                                     ? 1
                                     : 0;
  };
  if (!t || head_dim < 0 || heads < 0) return SWRT_E_INVALID_ARG;
  if (head_dim > INT32_MAX || heads > INT32_MAX) return SWRT_E_UNSUPPORTED;  // products below fit
  if (t->in_type != SWRT_XF_F32 && t->in_type != SWRT_XF_F16 && t->in_type != SWRT_XF_BF16)
    return SWRT_E_INVALID_ARG;
  if (bytes(t->out_type) == 0) return SWRT_E_INVALID_ARG;
  if ((t->cos_table == nullptr) != (t->sin_table == nullptr)) return SWRT_E_INVALID_ARG;
  *x = RowXf{};
  x->in_type = t->in_type;
  x->out_type = t->out_type;
  x->in_bytes = bytes(t->in_type);
  x->out_bytes = bytes(t->out_type);
  if (t->cos_table) {
    int64_t n;
    if (t->max_position < 1 || t->rotary_dim < 2 || t->rotary_dim % 2 ||
        t->rotary_dim > head_dim)
      return SWRT_E_INVALID_ARG;
    if (addr_of(t->cos_table) % 4 || addr_of(t->sin_table) % 4) return SWRT_E_INVALID_ARG;
    if (!mul_ok(t->max_position, t->rotary_dim / 2 * 4, &n)) return SWRT_E_UNSUPPORTED;
    ranges[(*nr)++] = range(t->cos_table, uint64_t(n), false);
    ranges[(*nr)++] = range(t->sin_table, uint64_t(n), false);
    x->cos = t->cos_table;
    x->sin = t->sin_table;
    x->max_pos = t->max_position;
    x->half = int32_t(t->rotary_dim / 2);
    x->interleaved = t->interleaved ? 1 : 0;
  }
  const bool fp8 = t->out_type == SWRT_XF_FP8_E4M3, affine = x->out_bytes == 1 && !fp8;
  if (x->out_bytes == 1) {
    x->lo = t->out_type == SWRT_XF_INT8 ? -128 : 0;
    x->hi = t->out_type == SWRT_XF_INT8 ? 127 : 255;
    for (int k = 0; k < 2; ++k) {
      const float sc = t->scale[k];
      if (!(sc > 0.0f) || sc > 3.4028235e38f) return SWRT_E_INVALID_ARG;  // positive, finite
      if (affine ? (t->zero_point[k] < x->lo || t->zero_point[k] > x->hi) : t->zero_point[k] != 0)
        return SWRT_E_INVALID_ARG;
      x->scale[k] = sc;
      x->zero[k] = t->zero_point[k];
    }
  }
  // per-channel tables [heads, head_dim]: scales of the byte targets, zero
  // points of the affine ones; their values are data (not checked here)
  int64_t tb = 0;
  const bool any = t->channel_scale[0] || t->channel_scale[1] || t->channel_zero_point[0] ||
                   t->channel_zero_point[1];
  if (any && !mul_ok(heads, head_dim * 4, &tb)) return SWRT_E_UNSUPPORTED;
  for (int k = 0; k < 2; ++k) {
    if ((t->channel_scale[k] && x->out_bytes != 1) || (t->channel_zero_point[k] && !affine))
      return SWRT_E_INVALID_ARG;
    if (addr_of(t->channel_scale[k]) % 4 || addr_of(t->channel_zero_point[k]) % 4)
      return SWRT_E_INVALID_ARG;
    if (t->channel_scale[k]) ranges[(*nr)++] = range(t->channel_scale[k], uint64_t(tb), false);
    if (t->channel_zero_point[k])
      ranges[(*nr)++] = range(t->channel_zero_point[k], uint64_t(tb), false);
    x->cs[k] = t->channel_scale[k];
    x->cz[k] = t->channel_zero_point[k];
  }
  x->d = int32_t(head_dim);
  x->heads = int32_t(heads > 0 ? heads : 1);
  return SWRT_OK;
}

}  // namespace swrt
