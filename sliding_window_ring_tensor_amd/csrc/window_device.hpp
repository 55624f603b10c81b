// window_device.hpp -- device bodies of the windowed GQA cache step.
//
// onnxruntime pull request "GQA support sliding_window_cache", section
// "Design": a windowed cache of capacity C keeps the L = min(T, C) most recent
// tokens at rows [0, L) of every (b, h) slice. Appending S tokens onto a past
// of P tokens, with Lp = min(P, C) resident and E = max(0, Lp + S - C)
// evicted, shifts cache[E .. Lp) to cache[0 .. Lp-E) and writes the new rows
// to cache[Lp-E .. Lp-E+S). Decode (S = 1) runs in place; any S > 1 step goes
// through a C+S staging cache that is copied back.
//
// Used by kv_seq_lengths.hip, kv_window.hip and decode_step.hip.
#pragma once

#include "xf_device.hpp"

namespace swrt {

// Workgroup shape of the window kernels: 512 threads (8 wave64s) moving two
// 16-byte words each per tile, i.e. one 16 KiB tile. Measured on MI355X for
// the decode step (C = 128, D = 64, bf16: one 16 KiB slice per workgroup):
// 512 x 2 beat 256 x 4, 128 x 8, 1024 x 1 and the 8 KiB tiles.
#ifndef SWRT_WIN_BLOCK
#define SWRT_WIN_BLOCK 512
#endif
#ifndef SWRT_WINDOW_UNROLL
#define SWRT_WINDOW_UNROLL 2
#endif
constexpr int kWinBlock = SWRT_WIN_BLOCK;
constexpr int kWinUnroll = SWRT_WINDOW_UNROLL;  // words per thread per tile
constexpr uint32_t kWinTile = kWinBlock * kWinUnroll;

// Element i of a per-batch length array that no kernel of the launch writes
// (seqlens_k, or Lp and E from an earlier launch), at an index equal on every
// lane of the wave. Read through the constant address space, so the compiler
// issues a scalar load: it waits in the scalar cache's queue, not behind the
// CU's vector memory traffic.
__device__ __forceinline__ int32_t ld_invariant(const int32_t *p, uint32_t i) {
  typedef const __attribute__((address_space(4))) int32_t *ConstPtr;
  return ((ConstPtr)p)[i];  // an address space cast (the C form is the one allowed)
}

// ---------------------------------------------------------------------------
// lengths of one step (same page, section "Design"; the follow-up commit does
// the arithmetic in 64 bits because seqlens_k + 1 overflows 32 bits at
// INT32_MAX, and clamps the past length at zero).
//
// The resident count after x tokens is end(x). The base layout keeps
// end(x) = min(x, C). The drifting layout of the CPU follow-up ("Key design
// decisions") lets the append point drift: with gap = C - W + 1, end(x) = x
// while x <= C, afterwards x minus as many whole gaps as bring it back to at
// most C (so W <= end <= C), which reclaims a whole gap at once, once every
// gap decode steps. gap = 1 is the base layout. A step appending S tokens
// onto P then has Lp = end(P), L = end(P + S) and E = Lp + S - L.
// ---------------------------------------------------------------------------
struct StepLengths {
  int64_t T, P, Lp, E, L;
  bool bad;  // seqlens_k < 0 or T < S
};

// x <= max(seqlens_k + 1, S) <= 2^31, so the ceiling quotient's numerator
// x - C + gap - 1 = x - W stays below 2^31 and the launch-wide divider applies.
__device__ __forceinline__ int64_t resident_end(int64_t x, int64_t C, const FastDiv &gap) {
  if (x <= C) return x;
  return x - int64_t(gap.d) * gap.div(uint32_t(x - C + gap.d - 1));
}

// DRIFT = false is the base layout (gap 1, end(x) = min(x, C)) without the
// division; DRIFT = true takes the gap from the launch.
template <bool DRIFT = true>
__device__ __forceinline__ StepLengths step_lengths(int32_t seqlens_k, int64_t S, int64_t C,
                                                    const FastDiv &gap) {
  StepLengths r;
  r.T = int64_t(seqlens_k) + 1;  // absolute total length after the step
  r.P = r.T - S;                  // absolute past length, clamped at zero
  if (r.P < 0) r.P = 0;
  if constexpr (DRIFT) {
    r.Lp = resident_end(r.P, C, gap);     // tokens resident before the step
    r.L = resident_end(r.P + S, C, gap);  // tokens resident after the step
  } else {
    r.Lp = r.P < C ? r.P : C;
    r.L = r.P + S < C ? r.P + S : C;
  }
  r.E = r.Lp + S - r.L;  // tokens evicted by the step
  r.bad = seqlens_k < 0 || r.T < S;
  return r;
}

// ---------------------------------------------------------------------------
// geometry shared by every slice of a launch
// ---------------------------------------------------------------------------
struct WindowGeom {
  const int32_t *lp, *ev;    // Lp, E per batch entry (null when derived in-kernel)
  const int64_t *past;       // absolute past lengths, the fused append's positions
  uint32_t *flags;
  int64_t nb_b, nb_h, nb_s;  // new-row strides, bytes
  uint64_t row_bytes;
  uint32_t H, BH, tiles, row_words;
  uint32_t slices;           // (layer, tensor, b, h) slices of the launch
  int32_t C, S;
  FastDiv by_row;            // words of the new part -> row (staging)
};

struct Slice {
  uint32_t layer, t, b, h;
};

// slice index -> (layer, tensor, b, h); h fastest, so consecutive workgroups
// walk consecutive slices of one cache
__device__ __forceinline__ Slice decode_slice(const WindowGeom &g, uint32_t slice) {
  const uint32_t lt = slice / g.BH, bh = slice - lt * g.BH;
  Slice s;
  s.layer = lt >> 1;
  s.t = lt & 1;
  s.b = bh / g.H;
  s.h = bh - s.b * g.H;
  return s;
}

// (Lp, E) must describe a step that fits the cache: 0 <= Lp <= C, E >= 0 and
// 1 <= L = Lp + S - E <= C (the base lengths and the drifting layout's both
// do). Otherwise flag once per batch entry (by the leader lane of the
// (layer 0, K, h 0) slice's first tile) and skip it.
__device__ __forceinline__ bool lengths_ok(const WindowGeom &g, const Slice &s, bool leader,
                                           int64_t Lp, int64_t E) {
  const int64_t L = Lp + g.S - E;
  if (Lp >= 0 && Lp <= g.C && E >= 0 && L >= 1 && L <= g.C) return true;
  if (g.flags && s.layer == 0 && s.t == 0 && s.h == 0 && leader)
    atomicOr(g.flags, SWRT_FLAG_BAD_LENGTHS);
  return false;
}

// Fused append: the entry's positions [P, P + S) must have table rows.
// Otherwise flag once per batch entry and skip it (the lengths were checked
// first).
__device__ __forceinline__ bool positions_ok(const WindowGeom &g, const RowXf &x, const Slice &s,
                                             bool leader, int64_t P) {
  if (xf_positions_ok(x, P, g.S)) return true;
  if (g.flags && s.layer == 0 && s.t == 0 && s.h == 0 && leader)
    atomicOr(g.flags, SWRT_FLAG_ROPE_RANGE);
  return false;
}

// ---------------------------------------------------------------------------
// S = 1, in place: one workgroup (BLOCK threads, UNROLL words each per tile)
// shifts one slice by E rows and appends the new row at Lp - E.
//
// The shift is an overlapping move with dst < src. The workgroup walks the
// slice in ascending tiles and, per tile, loads every word into registers,
// meets at a barrier, then stores: a later tile only reads rows above
// everything written so far, and a tile only overwrites rows whose old values
// its own loads already returned. No other workgroup touches the slice and no
// scratch memory is needed. Lanes past the end of the last tile clamp to its
// last word (same value to the same address as the owning lane), so the loop
// has no per-lane branch and the wait counters stay exact. With a one-wave
// workgroup the barrier compiles to nothing: the wave's vector memory
// operations take effect in issue order, and every store is issued after the
// load of its address, which keeps the same guarantee.
// ---------------------------------------------------------------------------
//
// XF: the appended row is the transform *xf of new_row (tensor t, absolute
// position pos) instead of a copy.
template <int VEC, int BLOCK = kWinBlock, int UNROLL = kWinUnroll, bool XF = false>
__device__ __forceinline__ void shift_append_slice(char *base, const char *new_row, int64_t Lp,
                                                   int64_t E, uint64_t row_bytes,
                                                   uint32_t row_words, const RowXf *xf = nullptr,
                                                   int t = 0, int64_t pos = 0, uint32_t h = 0) {
  using W = typename Word<VEC>::T;
  W *dst = reinterpret_cast<W *>(base);
  // The new row lives in its own buffer: fetch it first so its latency
  // overlaps the shift; it is stored at row Lp - E. (XF: its elements, one
  // or a few per lane, as XfLanes, in the waves that hold some.)
  const W *nsrc = reinterpret_cast<const W *>(new_row);
  W *adst = reinterpret_cast<W *>(base + uint64_t(Lp - E) * row_bytes);
  const bool row_in_one_pass = XF || row_words <= uint32_t(BLOCK);
  const uint32_t ai = min(threadIdx.x, row_words - 1);
  W nv;
  XfLanes<> xl;
  uint32_t D = 0;
  // XF: the row's loads go out right after the first tile's (or alone when
  // nothing shifts), never ahead of a wait the shift's addresses need
  if constexpr (XF)
    D = uint32_t(row_bytes) / uint32_t(xf->out_bytes);
  else if (row_in_one_pass)
    nv = ld(nsrc + ai);
  const bool row_wave = (threadIdx.x & ~63u) < D;  // uniform in a wave
  const auto append = [&]() {
    if constexpr (XF) {
      if (row_wave) {
        xf_lanes_encode(xl, *xf, t, threadIdx.x, BLOCK, D);
        xf_lanes_put(xl, *xf, reinterpret_cast<char *>(adst), threadIdx.x, BLOCK, D);
      }
    } else {
      st(adst + ai, nv);
    }
  };
  bool appended = false;
  if (E) {
    const W *src = reinterpret_cast<const W *>(base + uint64_t(E) * row_bytes);
    const uint32_t n = uint32_t(Lp - E) * row_words;
    for (uint32_t c0 = 0; c0 < n; c0 += uint32_t(BLOCK * UNROLL)) {
      W v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) v[u] = ld(src + min(c0 + u * BLOCK + threadIdx.x, n - 1));
      if constexpr (XF) {
        if (c0 == 0 && row_wave) {
          xf_lanes_load(xl, *xf, t, h, new_row, pos, threadIdx.x, BLOCK, D);
          xf_lanes_hold(xl);
        }
      }
      __syncthreads();  // every old value of this tile is in registers
      // Row Lp - E is no shift destination, and from here on every load of
      // every tile (this last one's included) has returned: the new row can
      // go out now, before the tile's stores, so that no work follows them
      // (work after a store that reuses its registers waits for the store to
      // complete).
      const bool last = row_in_one_pass && c0 + uint32_t(BLOCK * UNROLL) >= n;
      if (last) {
        append();
        appended = true;
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) st(dst + min(c0 + u * BLOCK + threadIdx.x, n - 1), v[u]);
    }
  }
  if (!appended) {  // no shift, or a row wider than one pass: after every load
    if (row_in_one_pass) {
      if constexpr (XF) {
        if (row_wave) xf_lanes_load(xl, *xf, t, h, new_row, pos, threadIdx.x, BLOCK, D);
      }
      append();
    } else {
      for (uint32_t i = threadIdx.x; i < row_words; i += BLOCK) st(adst + i, ld(nsrc + i));
    }
  }
}

// ---------------------------------------------------------------------------
// Shape of the one-wave variant: under the drifting layout most slices of a
// decode step only append their new row, so the step is many short
// workgroups; 64-thread workgroups (one wave, 16 words per lane) let 32 of
// them share a CU where 512-thread ones allow 4.
constexpr int kWaveBlock = 64;
constexpr int kWaveUnroll = 16;

// ---------------------------------------------------------------------------
// S = 1, in place, several small slices per workgroup. When a whole slice is
// at most one tile of a subgroup (kWinBlock / SPW threads), the workgroup is
// split into SPW subgroups of whole waves, one slice each, meeting at a single
// shared barrier: loads of every subgroup, barrier, stores. The same ordering
// argument as shift_append_slice holds inside each slice; slices never share
// rows. `info(slice, g)` returns the work of subgroup g's slice (ok = false:
// leave it alone); each wave evaluates it for its own subgroup only, in
// uniform code, so its table lookups stay scalar.
// ---------------------------------------------------------------------------
struct SliceWork {
  char *base;           // row 0 of the slice
  const char *new_row;  // the appended row
  int64_t Lp, E;
  int64_t pos;          // its absolute position (fused append)
  int t;                // 0 = K, 1 = V
  uint32_t h;           // its KV head (per-channel parameters)
  bool ok;
};

// the work of one wave's slice, its integers taken from the first lane (they
// are equal on every lane of the wave; the pointers stay as they are, so the
// compiler keeps their global address space)
__device__ __forceinline__ SliceWork wave_uniform(const SliceWork &w) {
  SliceWork u = w;
  u.Lp = int64_t(uniform_u64(uint64_t(w.Lp)));
  u.E = int64_t(uniform_u64(uint64_t(w.E)));
  u.pos = int64_t(uniform_u64(uint64_t(w.pos)));
  u.t = __builtin_amdgcn_readfirstlane(w.t);
  u.h = uint32_t(__builtin_amdgcn_readfirstlane(int32_t(w.h)));
  u.ok = __builtin_amdgcn_readfirstlane(int32_t(w.ok)) != 0;
  return u;
}

#ifndef SWRT_GROUP_UNROLL
#define SWRT_GROUP_UNROLL 2
#endif
constexpr int kGroupUnroll = SWRT_GROUP_UNROLL;  // words per lane per slice in group mode
// A fused append's subgroup takes as many words a lane as a plain copy's. Four
// (twice the slices per workgroup, to hide the row's few dependent steps:
// loads, arithmetic, store) measured slower once each wave works out only its
// own slice: 35.6 against 34.8 us on a 24-layer int8 fused decode step.
constexpr int kGroupUnrollXf = 2;
template <bool XF>
constexpr int group_unroll() { return XF ? kGroupUnrollXf : kGroupUnroll; }

template <int VEC, int SPW, bool XF = false, typename Info>
__device__ __forceinline__ void shift_append_group(uint32_t first_slice, uint32_t n_slices,
                                                   uint64_t row_bytes, uint32_t row_words,
                                                   Info info, const RowXf *xf = nullptr) {
  using W = typename Word<VEC>::T;
  constexpr uint32_t GB = kWinBlock / SPW;  // threads per subgroup (a multiple of 64)
  static_assert(GB % 64 == 0, "subgroups must be whole waves");
  // A subgroup is whole waves: the subgroup index is uniform in a wave, so each
  // wave works out its own slice alone, in scalar code (its table lookups are
  // scalar loads); the slice's work then stays in scalar registers, so that
  // what it selects (a tensor's table pointers among the kernel arguments) is
  // a scalar load, not a vector load whose wait would also drain the shift's
  // loads issued before it.
  const uint32_t lid = threadIdx.x % GB;
  const uint32_t grp = uint32_t(__builtin_amdgcn_readfirstlane(int32_t(threadIdx.x / GB)));
  SliceWork w;
  w.ok = false;
  if (first_slice + grp < n_slices) w = info(first_slice + grp, int(grp));
  w = wave_uniform(w);
  // n, the words to shift, and w.ok are uniform inside a subgroup, so the two
  // predicated blocks below never split a wave. A slice with nothing to shift
  // (E = 0) points its shift words at the appended row: the same value to the
  // same address. Loads and stores then each form one straight block, which
  // keeps the wait counters exact (stores are never held behind other stores).
  const uint32_t n = (w.ok && w.E) ? uint32_t(w.Lp - w.E) * row_words : 0;
  const uint32_t ai = min(lid, row_words - 1);
  const W *nsrc = reinterpret_cast<const W *>(w.new_row) + ai;
  W *adst = reinterpret_cast<W *>(w.base + uint64_t(w.Lp - w.E) * row_bytes) + ai;
  const W *src = reinterpret_cast<const W *>(w.base + uint64_t(w.E) * row_bytes);
  W *dst = reinterpret_cast<W *>(w.base);
  constexpr int GU = group_unroll<XF>();
  W v[GU], nv;
  XfLanes<1> xl;  // a row of a fused group fits its subgroup's lanes
  const uint32_t D = XF ? uint32_t(row_bytes) / uint32_t(xf->out_bytes) : 0;
  // the waves that hold elements of the appended row (uniform in a wave): the
  // others of the subgroup only shift
  const bool row_wave = (lid & ~63u) < D;
  if (w.ok) {
    if constexpr (XF) {
      // the appended row is transformed, not copied: a slice with nothing to
      // shift (n = 0, uniform in the subgroup) moves no words at all; the
      // row's loads follow the shift's (no wait for them precedes a shift load)
      if (n) {
#pragma unroll
        for (int u = 0; u < GU; ++u) v[u] = ld(src + min(u * GB + lid, n - 1));
      }
      if (row_wave) {
        xf_lanes_load(xl, *xf, w.t, w.h, w.new_row, w.pos, lid, GB, D);
        xf_lanes_hold(xl);
      }
    } else {
      nv = ld(nsrc);
#pragma unroll
      for (int u = 0; u < GU; ++u) v[u] = ld(n ? src + min(u * GB + lid, n - 1) : nsrc);
    }
  }
  __syncthreads();  // every old value of every slice of the workgroup is in registers
  if (w.ok) {
    if constexpr (XF) {
      // the row first, so that nothing follows the shift's stores (work after
      // a store that reuses its registers waits for the store to complete)
      if (row_wave) {
        xf_lanes_encode(xl, *xf, w.t, lid, GB, D);
        xf_lanes_put(xl, *xf, w.base + uint64_t(w.Lp - w.E) * row_bytes, lid, GB, D);
      }
      if (n) {
#pragma unroll
        for (int u = 0; u < GU; ++u) st(dst + min(u * GB + lid, n - 1), v[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < GU; ++u) st(n ? dst + min(u * GB + lid, n - 1) : adst, v[u]);
      st(adst, nv);
    }
  }
}

// Slices per workgroup for an in-place launch: the most (1, 2 or 4) whose
// subgroup tile still holds a whole shift and whose subgroup covers a row.
//
// A fused append (xf) gives each lane of the subgroup (kWinBlock / spw lanes)
// one element of the appended row, row_elems of them: the subgroup is also at
// least as wide as that row (wider rows take the one-slice shape, a few
// elements a lane). Its subgroups take group_unroll<true>() words a lane.
inline int slices_per_group(int64_t capacity, uint32_t row_words, bool xf = false,
                            int64_t row_elems = 0) {
  const uint64_t gu = xf ? group_unroll<true>() : group_unroll<false>();
  int spw = 1;
  while (spw < 4 &&
         uint64_t(capacity - 1) * row_words <= uint64_t(kWinBlock / (2 * spw)) * gu &&
         row_words <= uint32_t(kWinBlock / (2 * spw)) &&
         row_elems <= int64_t(kWinBlock / (2 * spw)))
    spw *= 2;
  return spw;
}

// S > 1, STAGE: tile `tile` of staging[0 .. Lp+S): words of rows [0, Lp) from
// the cache, of rows [Lp, Lp+S) from the (strided) new rows.
//
// XF: new row r is the transform *xf of the given row (tensor t, absolute
// position P + r).
template <int VEC, bool XF = false>
__device__ __forceinline__ void stage_tile(const WindowGeom &g, const char *cache_slice,
                                           char *stage_slice, const char *new_rows, int64_t Lp,
                                           uint32_t tile, const RowXf *xf = nullptr, int t = 0,
                                           int64_t P = 0, uint32_t h = 0) {
  using W = typename Word<VEC>::T;
  const uint32_t n_seed = uint32_t(Lp) * g.row_words;
  const uint32_t n = uint32_t(Lp + g.S) * g.row_words;
  const uint32_t i0 = tile * kWinTile;
  if (i0 >= n) return;
  const W *cache = reinterpret_cast<const W *>(cache_slice);
  W *stage = reinterpret_cast<W *>(stage_slice);
  W v[kWinUnroll];
#pragma unroll
  for (int u = 0; u < kWinUnroll; ++u) {
    const uint32_t i = min(i0 + u * kWinBlock + threadIdx.x, n - 1);  // tail lanes repeat the last word
    const uint32_t j = i < n_seed ? 0 : i - n_seed, r = g.by_row.div(j), c = j - r * g.row_words;
    if constexpr (XF) {
      v[u] = i < n_seed ? ld(cache + i)
                        : xf_word<VEC>(*xf, t, h, new_rows + int64_t(r) * g.nb_s, P + r, c);
    } else {
      const W *p = i < n_seed ? cache + i : reinterpret_cast<const W *>(new_rows + int64_t(r) * g.nb_s) + c;
      v[u] = ld(p);
    }
  }
#pragma unroll
  for (int u = 0; u < kWinUnroll; ++u) st(stage + min(i0 + u * kWinBlock + threadIdx.x, n - 1), v[u]);
}

// S > 1, COMMIT: tile `tile` of cache[0 .. L) <- staging[E .. E+L), or of rows
// [Lp, L) only when nothing was evicted (rows below Lp of staging are the
// cache's own rows).
template <int VEC>
__device__ __forceinline__ void commit_tile(const WindowGeom &g, char *cache_slice,
                                            const char *stage_slice, int64_t Lp, int64_t E,
                                            uint32_t tile) {
  using W = typename Word<VEC>::T;
  const int64_t L = Lp + g.S - E;
  const int64_t r0 = E ? 0 : Lp;
  const uint32_t n = uint32_t(L - r0) * g.row_words;
  const uint32_t i0 = tile * kWinTile;
  if (i0 >= n) return;
  W *dst = reinterpret_cast<W *>(cache_slice + uint64_t(r0) * g.row_bytes);
  const W *src = reinterpret_cast<const W *>(stage_slice + uint64_t(E + r0) * g.row_bytes);
  W v[kWinUnroll];
#pragma unroll
  for (int u = 0; u < kWinUnroll; ++u) v[u] = ld(src + min(i0 + u * kWinBlock + threadIdx.x, n - 1));
#pragma unroll
  for (int u = 0; u < kWinUnroll; ++u) st(dst + min(i0 + u * kWinBlock + threadIdx.x, n - 1), v[u]);
}

}  // namespace swrt
