// scatter_device.hpp -- device bodies of TensorScatter (ONNX operator page
// "TensorScatter", ai.onnx since version 24: description, pseudocode,
// Attributes).
//
// The cache is viewed as [O, M, I]: O = product of the dims before `axis`,
// M = shape[axis] (max_sequence_length), I = product of the dims after it; the
// update is [O, S, I]; prefix o belongs to batch entry b = o / (O / B). Row
// (o, s) of the update goes to cache row j = w_b + s (linear) or
// (w_b + s) mod M (circular, floor modulo, applied to the sequence index
// only). A linear entry with w_b < 0 or w_b > M - S is flagged and its rows
// keep past's values.
//
// Used by tensor_scatter.hip and decode_step.hip. The XF instances are the
// fused append (xf_device.hpp): update rows pass through the row transform at
// absolute positions w_b + s (before the circular wrap), and entries whose
// positions leave the rotary tables are flagged and skipped like linear
// out-of-range ones.
#pragma once

#include "xf_device.hpp"

namespace swrt {

// Standalone scatter kernels run 128-thread workgroups of 4 words per thread
// (8 KiB tiles): on MI355X smaller tiles stream better here (a 1 GiB copy
// through the out-of-place kernel: 6.46 TB/s at 128 threads, 6.37 at 256,
// 6.30 at 512). The one-launch decode step reuses these bodies at its own
// workgroup size, so they take the block size as a template argument.
#ifndef SWRT_SCAT_BLOCK
#define SWRT_SCAT_BLOCK 128
#endif
constexpr int kScatBlock = SWRT_SCAT_BLOCK;
constexpr int kScatUnroll = 4;  // words per thread per tile

struct ScatterGeom {
  const int64_t *write_indices;  // [B] or null (zeros)
  uint32_t *flags;
  int64_t M, S;
  uint32_t n_words;        // words per tensor: update words in place, present words otherwise
  uint32_t words_per_row;  // row bytes / VEC
  FastDiv by_row;          // word -> row
  FastDiv by_seq;          // row -> (o, s) in place; row -> (o, j) out of place
  FastDiv by_batch;        // o -> b
  int circular;
  uint32_t in_row_bytes;   // fused append: bytes of an update row (in_type)
};

// floor modulo of a 64-bit index into [0, M); the division is skipped for the
// usual case of an index already in range.
__device__ __forceinline__ int64_t wrap_index(int64_t w, int64_t M) {
  if (w >= 0 && w < M) return w;
  int64_t r = w % M;
  return r < 0 ? r + M : r;
}

// The write index of every batch entry a tile touches, staged once in LDS (a
// tile's words span at most TILE + 1 entries). Circular entries hold
// w mod M; linear entries hold w, or -1 when the entry is out of range (then
// flagged). Lane lookups are LDS reads, so the only global loads of a lane are
// its payload words.
template <uint32_t TILE, bool RAW = false>
struct TileBatches {
  uint32_t first;
  int64_t w[TILE + 1];
  int64_t raw[RAW ? TILE + 1 : 1];  // fused append: w before the wrap (the position)
};

__device__ __forceinline__ int64_t reduce_write_index(const ScatterGeom &g, int64_t w) {
  if (g.circular) return wrap_index(w, g.M);
  if (w < 0 || w > g.M - g.S) {  // no partial update of this batch entry
    if (g.flags) atomicOr(g.flags, SWRT_FLAG_LINEAR_OOB);
    return -1;
  }
  return w;
}

// Staging runs in two halves around the payload loads: the first half issues
// the index loads (thread k fetches entry first + k), the second waits for
// them, fills LDS and meets at a barrier. Vector memory counters retire in
// order, so index loads issued before the payload loads are waited for
// without waiting for the payload.
struct WPrefetch {
  uint32_t first, count;
  int64_t w;
};

template <int BLOCK>
__device__ __forceinline__ WPrefetch prefetch_write_indices(const ScatterGeom &g, uint32_t tile) {
  const uint32_t last = min(tile + uint32_t(BLOCK * kScatUnroll), g.n_words) - 1;
  WPrefetch p;
  p.first = g.by_batch.div(g.by_seq.div(g.by_row.div(tile)));
  p.count = g.by_batch.div(g.by_seq.div(g.by_row.div(last))) - p.first + 1;
  const uint32_t k = min(threadIdx.x, p.count - 1);
  p.w = g.write_indices ? g.write_indices[p.first + k] : 0;
  return p;
}

// fused append: a valid entry must also have its positions in the tables
__device__ __forceinline__ int64_t reduce_write_index_xf(const ScatterGeom &g, const RowXf &x,
                                                         int64_t w) {
  const int64_t r = reduce_write_index(g, w);
  if (r < 0 || xf_positions_ok(x, w, g.S)) return r;
  if (g.flags) atomicOr(g.flags, SWRT_FLAG_ROPE_RANGE);
  return -1;
}

template <int BLOCK, uint32_t TILE, bool XF = false>
__device__ __forceinline__ void finish_write_indices(const ScatterGeom &g, const WPrefetch &p,
                                                     TileBatches<TILE, XF> &tb,
                                                     const RowXf *xf = nullptr) {
  const auto stage = [&](uint32_t k, int64_t w) {
    if constexpr (XF) {
      tb.w[k] = reduce_write_index_xf(g, *xf, w);
      tb.raw[k] = w;
    } else {
      tb.w[k] = reduce_write_index(g, w);
    }
  };
  if (threadIdx.x == 0) tb.first = p.first;
  if (threadIdx.x < p.count) stage(threadIdx.x, p.w);
  for (uint32_t k = threadIdx.x + BLOCK; k < p.count; k += BLOCK)  // many tiny rows
    stage(k, g.write_indices ? g.write_indices[p.first + k] : 0);
  __syncthreads();
}

// In place: tile `tile` (a word offset) of the update moves to its cache rows.
// Lanes past the last word clamp to it (repeating that lane's load and store),
// so only the linear out-of-range skip guards stores. XF: each word is the
// transform of update row (o, s) at position w + s (tensor t), computed once
// the write indices are staged.
template <int VEC, int BLOCK, bool XF = false>
__device__ __forceinline__ void scatter_in_place_tile(const ScatterGeom &g, char *present_,
                                                      const char *update_, uint32_t tile,
                                                      TileBatches<BLOCK * kScatUnroll, XF> &tb,
                                                      const RowXf *xf = nullptr, int t = 0) {
  using W = typename Word<VEC>::T;
  const WPrefetch wp = prefetch_write_indices<BLOCK>(g, tile);
  const W *update = reinterpret_cast<const W *>(update_);
  W *present = reinterpret_cast<W *>(present_);
  W v[kScatUnroll];
  if constexpr (!XF) {
#pragma unroll
    for (int u = 0; u < kScatUnroll; ++u) v[u] = ld(update + min(tile + u * BLOCK + threadIdx.x, g.n_words - 1));
  }
  finish_write_indices<BLOCK>(g, wp, tb, xf);
#pragma unroll
  for (int u = 0; u < kScatUnroll; ++u) {
    const uint32_t i = min(tile + u * BLOCK + threadIdx.x, g.n_words - 1);
    const uint32_t row = g.by_row.div(i);
    const uint32_t col = i - row * g.words_per_row;
    const uint32_t o = g.by_seq.div(row);
    const uint32_t s = row - o * uint32_t(g.S);
    const uint32_t k = g.by_batch.div(o) - tb.first;
    const int64_t w = tb.w[k];
    int64_t j = w + s;
    if (g.circular && j >= g.M) j -= g.M;
    if (w >= 0) {
      if constexpr (XF) {
        const uint32_t h = xf_channels(*xf) ? o % uint32_t(xf->heads) : 0;  // KV head of the row
        v[u] = xf_word<VEC>(*xf, t, h, update_ + uint64_t(row) * g.in_row_bytes, tb.raw[k] + s,
                            col);
      }
      st(present + (int64_t(o) * g.M + j) * g.words_per_row + col, v[u]);
    }
  }
}

// Out of place: tile `tile` of present, every word from past or the update.
template <int VEC, int BLOCK, bool XF = false>
__device__ __forceinline__ void scatter_out_of_place_tile(const ScatterGeom &g, char *present_,
                                                          const char *past_, const char *update_,
                                                          uint32_t tile,
                                                          TileBatches<BLOCK * kScatUnroll, XF> &tb,
                                                          const RowXf *xf = nullptr, int t = 0) {
  using W = typename Word<VEC>::T;
  finish_write_indices<BLOCK>(g, prefetch_write_indices<BLOCK>(g, tile), tb, xf);
  const W *update = reinterpret_cast<const W *>(update_);
  const W *past = reinterpret_cast<const W *>(past_);
  W *present = reinterpret_cast<W *>(present_);
  W v[kScatUnroll];
#pragma unroll
  for (int u = 0; u < kScatUnroll; ++u) {
    const uint32_t i = min(tile + u * BLOCK + threadIdx.x, g.n_words - 1);
    const uint32_t row = g.by_row.div(i);
    const uint32_t col = i - row * g.words_per_row;
    const uint32_t o = g.by_seq.div(row);
    const int64_t j = row - o * uint32_t(g.M);
    const uint32_t k = g.by_batch.div(o) - tb.first;
    const int64_t w = tb.w[k];
    int64_t s = -1;  // the update row landing on (o, j), if any
    if (w >= 0) {
      s = j - w;
      if (g.circular && s < 0) s += g.M;
      if (s >= g.S) s = -1;
    }
    if constexpr (XF) {
      const uint32_t h = xf_channels(*xf) ? o % uint32_t(xf->heads) : 0;  // KV head of the row
      v[u] = s >= 0 ? xf_word<VEC>(*xf, t, h, update_ + (uint64_t(o) * g.S + s) * g.in_row_bytes,
                                   tb.raw[k] + s, col)
                    : ld(past + i);
    } else {
      v[u] = ld(s >= 0 ? update + (int64_t(o) * g.S + s) * g.words_per_row + col : past + i);
    }
  }
#pragma unroll
  for (int u = 0; u < kScatUnroll; ++u) st(present + min(tile + u * BLOCK + threadIdx.x, g.n_words - 1), v[u]);
}

}  // namespace swrt
