// kv_window.hip -- the windowed GQA cache step on gfx950.
//
// onnxruntime pull request "GQA support sliding_window_cache", section
// "Design". A windowed cache of capacity C keeps the L = min(T, C) most recent
// tokens at rows [0, L) of every (b, h) slice. Appending S tokens onto a past
// of P tokens, with Lp = min(P, C) resident and E = max(0, Lp + S - C)
// evicted, shifts cache[E .. Lp) to cache[0 .. Lp-E) and writes the new rows
// to cache[Lp-E .. Lp-E+S). Decode (S = 1) runs in place, shifting at most one
// row; any S > 1 step is seeded into a C+S staging cache and the surviving
// window is copied back, for K and V in one launch each.
//
// Kernels (K and V of every layer in the same launch, one slice = one (layer,
// tensor, b, h); consecutive workgroups walk consecutive slices in memory):
//   window_in_place  S = 1. One workgroup per slice. The shift is an
//                    overlapping move with dst < src, so the workgroup walks
//                    the slice in ascending tiles and, per tile, loads every
//                    word into registers, meets at a barrier, then stores:
//                    a later tile only reads rows above everything already
//                    written, and a tile only overwrites rows all of whose old
//                    values its own loads have returned. The appended row goes
//                    last, after the final barrier (with E = 1 it overwrites a
//                    row the shift read). Configurations with C = 128 rows of
//                    64 bf16 take one tile: 16 KiB in, 16 KiB out.
//   window_stage     S > 1, phase STAGE. Tiles of the staging slice; words of
//                    rows [0, Lp) come from the cache, rows [Lp, Lp+S) from
//                    the new tokens (strided rows, head_dim contiguous).
//   window_commit    S > 1, phase COMMIT. cache[0 .. L) <- staging[E .. E+L),
//                    or only rows [Lp, L) when nothing was evicted (rows below
//                    Lp of staging are the cache's own rows).
// Batch entries whose (Lp, E) pair is not the one the lengths define for
// (C, S) are flagged and left untouched.
#include "swrt_device.hpp"

namespace swrt {
namespace {

#ifndef SWRT_WINDOW_UNROLL
#define SWRT_WINDOW_UNROLL 4
#endif
constexpr int kUnroll = SWRT_WINDOW_UNROLL;  // words per thread per tile
constexpr int kMaxLayers = SWRT_MAX_LAYERS;  // layers per batched launch

template <int NL>
struct WinArgs {
  char *cache[NL][2];
  const char *nw[NL][2];
  char *stage[NL][2];
  const int32_t *lp, *ev;
  uint32_t *flags;
  int64_t nb_b, nb_h, nb_s;  // new-row strides, bytes
  uint64_t row_bytes;
  uint32_t H, BH, tiles, row_words;
  int32_t C, S;
  FastDiv by_row;  // words of the new part -> row
};

struct Slice {
  uint32_t layer, t, b, h;
};

template <int NL>
__device__ __forceinline__ Slice decode(const WinArgs<NL> &a, uint32_t slice) {
  const uint32_t lt = slice / a.BH, bh = slice - lt * a.BH;
  Slice s;
  s.layer = lt >> 1;
  s.t = lt & 1;
  s.b = bh / a.H;
  s.h = bh - s.b * a.H;
  return s;
}

// (Lp, E) must be what the lengths give for (C, S): 0 <= Lp <= C and
// E = max(0, Lp + S - C). Otherwise flag once per batch entry and skip.
template <int NL>
__device__ __forceinline__ bool lengths_ok(const WinArgs<NL> &a, const Slice &s, uint32_t tile,
                                           int64_t Lp, int64_t E) {
  int64_t e = Lp + a.S - a.C;
  if (e < 0) e = 0;
  if (Lp >= 0 && Lp <= a.C && E == e) return true;
  if (a.flags && s.layer == 0 && s.t == 0 && s.h == 0 && tile == 0 && threadIdx.x == 0)
    atomicOr(a.flags, SWRT_FLAG_BAD_LENGTHS);
  return false;
}

template <int VEC, int NL>
__global__ __launch_bounds__(kBlock) void window_in_place(WinArgs<NL> a) {
  using W = typename Word<VEC>::T;
  const Slice s = decode(a, blockIdx.x);
  const int64_t Lp = a.lp[s.b], E = a.ev[s.b];
  if (!lengths_ok(a, s, 0, Lp, E)) return;

  char *base = a.cache[s.layer][s.t] + uint64_t(s.b * a.H + s.h) * uint64_t(a.C) * a.row_bytes;
  W *dst = reinterpret_cast<W *>(base);
  // The new row lives in its own buffer: fetch it first so its latency
  // overlaps the shift. It is stored last, at row Lp - E.
  const W *nsrc = reinterpret_cast<const W *>(a.nw[s.layer][s.t] + s.b * a.nb_b + s.h * a.nb_h);
  W *adst = reinterpret_cast<W *>(base + uint64_t(Lp - E) * a.row_bytes);
  const bool row_in_one_pass = a.row_words <= kBlock;
  const uint32_t ai = min(threadIdx.x, a.row_words - 1);
  W nv;
  if (row_in_one_pass) nv = ld(nsrc + ai);
  bool appended = false;
  if (E) {
    // Lanes past the end of the last tile clamp to its last word: they load
    // and store the same value to the same address as the lane that owns it,
    // which keeps the loop free of per-lane branches.
    const W *src = reinterpret_cast<const W *>(base + uint64_t(E) * a.row_bytes);
    const uint32_t n = uint32_t(Lp - E) * a.row_words;
    for (uint32_t c0 = 0; c0 < n; c0 += kBlock * kUnroll) {
      W v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = ld(src + min(c0 + u * kBlock + threadIdx.x, n - 1));
      __syncthreads();  // every old value of this tile is in registers
      // Row Lp - E is read by the last tile and is no shift destination: the
      // new row can go out as soon as that tile's loads are done.
      if (row_in_one_pass && c0 + kBlock * kUnroll >= n) {
        st(adst + ai, nv);
        appended = true;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) st(dst + min(c0 + u * kBlock + threadIdx.x, n - 1), v[u]);
    }
  }
  if (!appended) {  // no shift, or a row wider than one pass: after every load
    if (row_in_one_pass) {
      st(adst + ai, nv);
    } else {
      for (uint32_t i = threadIdx.x; i < a.row_words; i += kBlock) st(adst + i, ld(nsrc + i));
    }
  }
}

template <int VEC, int NL>
__global__ __launch_bounds__(kBlock) void window_stage(WinArgs<NL> a) {
  using W = typename Word<VEC>::T;
  const uint32_t slice = blockIdx.x / a.tiles, tile = blockIdx.x - slice * a.tiles;
  const Slice s = decode(a, slice);
  const int64_t Lp = a.lp[s.b], E = a.ev[s.b];
  if (!lengths_ok(a, s, tile, Lp, E)) return;

  const uint32_t n_seed = uint32_t(Lp) * a.row_words;
  const uint32_t n = uint32_t(Lp + a.S) * a.row_words;
  const uint32_t i0 = tile * (kBlock * kUnroll);
  if (i0 >= n) return;
  const uint64_t bh = s.b * a.H + s.h;
  const W *cache = reinterpret_cast<const W *>(a.cache[s.layer][s.t] + bh * uint64_t(a.C) * a.row_bytes);
  W *stage = reinterpret_cast<W *>(a.stage[s.layer][s.t] + bh * uint64_t(a.C + a.S) * a.row_bytes);
  const char *nw = a.nw[s.layer][s.t] + s.b * a.nb_b + s.h * a.nb_h;
  W v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t i = min(i0 + u * kBlock + threadIdx.x, n - 1);  // tail lanes repeat the last word
    const uint32_t j = i < n_seed ? 0 : i - n_seed, r = a.by_row.div(j), c = j - r * a.row_words;
    const W *p = i < n_seed ? cache + i : reinterpret_cast<const W *>(nw + int64_t(r) * a.nb_s) + c;
    v[u] = ld(p);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) st(stage + min(i0 + u * kBlock + threadIdx.x, n - 1), v[u]);
}

template <int VEC, int NL>
__global__ __launch_bounds__(kBlock) void window_commit(WinArgs<NL> a) {
  using W = typename Word<VEC>::T;
  const uint32_t slice = blockIdx.x / a.tiles, tile = blockIdx.x - slice * a.tiles;
  const Slice s = decode(a, slice);
  const int64_t Lp = a.lp[s.b], E = a.ev[s.b];
  if (!lengths_ok(a, s, tile, Lp, E)) return;

  const int64_t L = Lp + a.S - E;
  const int64_t r0 = E ? 0 : Lp;  // with no eviction rows [0, Lp) are already in place
  const uint32_t n = uint32_t(L - r0) * a.row_words;
  const uint32_t i0 = tile * (kBlock * kUnroll);
  if (i0 >= n) return;
  const uint64_t bh = s.b * a.H + s.h;
  W *dst = reinterpret_cast<W *>(a.cache[s.layer][s.t] + (bh * uint64_t(a.C) + r0) * a.row_bytes);
  const W *src = reinterpret_cast<const W *>(
      a.stage[s.layer][s.t] + (bh * uint64_t(a.C + a.S) + E + r0) * a.row_bytes);
  W v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) v[u] = ld(src + min(i0 + u * kBlock + threadIdx.x, n - 1));
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) st(dst + min(i0 + u * kBlock + threadIdx.x, n - 1), v[u]);
}

template <int VEC, int NL>
int launch(WinArgs<NL> a, uint32_t slices, unsigned phase, hipStream_t stream) {
  const uint64_t tile_words = kBlock * kUnroll;
  if (a.S == 1) {
    hipLaunchKernelGGL((window_in_place<VEC, NL>), dim3(slices), dim3(kBlock), 0, stream, a);
    return launch_status();
  }
  if (phase & SWRT_PHASE_STAGE) {
    a.tiles = uint32_t((uint64_t(a.C + a.S) * a.row_words + tile_words - 1) / tile_words);
    hipLaunchKernelGGL((window_stage<VEC, NL>), dim3(slices * a.tiles), dim3(kBlock), 0, stream, a);
    if (launch_status() != SWRT_OK) return SWRT_E_LAUNCH;
  }
  if (phase & SWRT_PHASE_COMMIT) {
    a.tiles = uint32_t((uint64_t(a.C) * a.row_words + tile_words - 1) / tile_words);
    hipLaunchKernelGGL((window_commit<VEC, NL>), dim3(slices * a.tiles), dim3(kBlock), 0, stream, a);
    if (launch_status() != SWRT_OK) return SWRT_E_LAUNCH;
  }
  return SWRT_OK;
}

// Validation and launch shared by the single-layer and the batched entry point.
int window_append(int n_layers, void *const *k_caches, void *const *v_caches,
                  const void *const *k_news, const void *const *v_news,
                  const int64_t *new_strides, void *const *k_stagings, void *const *v_stagings,
                  const int32_t *cache_past_lens, const int32_t *evict_counts, int batch,
                  int kv_heads, int capacity, int seq_len, int head_dim, int elem_bits,
                  unsigned phase, uint32_t *d_flags, void *stream) {
  if (n_layers < 0 || n_layers > kMaxLayers) return SWRT_E_INVALID_ARG;
  if (batch < 0 || kv_heads < 0 || head_dim < 0 || capacity < 1 || seq_len < 1)
    return SWRT_E_INVALID_ARG;
  if (!valid_elem_bits(elem_bits)) return SWRT_E_INVALID_ARG;
  const int64_t B = batch, H = kv_heads, C = capacity, S = seq_len, D = head_dim;
  if (S > 1 && phase != SWRT_PHASE_STAGE && phase != SWRT_PHASE_COMMIT && phase != SWRT_PHASE_ALL)
    return SWRT_E_INVALID_ARG;
  if (!new_strides) return SWRT_E_INVALID_ARG;
  if ((D * elem_bits) % 8) return SWRT_E_UNSUPPORTED;
  int64_t nb[3];
  for (int i = 0; i < 3; ++i) {
    if (new_strides[i] < 0) return SWRT_E_INVALID_ARG;
    if (!mul_ok(new_strides[i], elem_bits, &nb[i]) || nb[i] % 8) return SWRT_E_UNSUPPORTED;
    nb[i] /= 8;
  }
  const int64_t row = D * elem_bits / 8;
  if (n_layers == 0 || B == 0 || H == 0 || row == 0) return SWRT_OK;
  if (!k_caches || !v_caches || !k_news || !v_news || !cache_past_lens || !evict_counts)
    return SWRT_E_INVALID_ARG;
  if (S > 1 && (!k_stagings || !v_stagings)) return SWRT_E_INVALID_ARG;

  // sizes, limits
  int64_t slices, cache_bytes, stage_bytes, t;
  if (!mul_ok(B * H, 2 * int64_t(n_layers), &slices) || slices >= (int64_t(1) << 31))
    return SWRT_E_UNSUPPORTED;
  if (!mul_ok(B * H * C, row, &cache_bytes) || !mul_ok(B * H * (C + S), row, &stage_bytes))
    return SWRT_E_UNSUPPORTED;
  const int64_t new_span = (B - 1) * nb[0] + (H - 1) * nb[1] + (S - 1) * nb[2] + row;

  const auto addr = [](const void *p) { return uint64_t(reinterpret_cast<uintptr_t>(p)); };
  const uint64_t align = elem_bits >= 16 ? uint64_t(elem_bits / 8 > 8 ? 8 : elem_bits / 8) : 1;
  if (addr(cache_past_lens) % 4 || addr(evict_counts) % 4 || addr(d_flags) % 4)
    return SWRT_E_INVALID_ARG;

  uint64_t align_acc = uint64_t(row) | uint64_t(nb[0]) | uint64_t(nb[1]) | uint64_t(nb[2]);
  WinArgs<kMaxLayers> a = {};
  // every buffer of every layer: non-null and aligned; caches, staging buffers
  // and the flag word are written, so nothing may overlap them (across layers
  // too); new rows and lengths are only read and may be shared.
  Range ranges[6 * kMaxLayers + 3];
  int nr = 0;
  for (int l = 0; l < n_layers; ++l) {
    const void *p[6] = {k_caches[l], v_caches[l], k_news[l], v_news[l],
                        S > 1 ? k_stagings[l] : nullptr, S > 1 ? v_stagings[l] : nullptr};
    const uint64_t n[6] = {uint64_t(cache_bytes), uint64_t(cache_bytes), uint64_t(new_span),
                           uint64_t(new_span), uint64_t(stage_bytes), uint64_t(stage_bytes)};
    for (int i = 0; i < (S > 1 ? 6 : 4); ++i) {
      if (!p[i] || addr(p[i]) % align) return SWRT_E_INVALID_ARG;
      align_acc |= addr(p[i]);
      ranges[nr++] = range(p[i], n[i], i != 2 && i != 3);
    }
    a.cache[l][0] = static_cast<char *>(k_caches[l]);
    a.cache[l][1] = static_cast<char *>(v_caches[l]);
    a.nw[l][0] = static_cast<const char *>(k_news[l]);
    a.nw[l][1] = static_cast<const char *>(v_news[l]);
    a.stage[l][0] = S > 1 ? static_cast<char *>(k_stagings[l]) : nullptr;
    a.stage[l][1] = S > 1 ? static_cast<char *>(v_stagings[l]) : nullptr;
  }
  ranges[nr++] = range(cache_past_lens, uint64_t(B) * 4, false);
  ranges[nr++] = range(evict_counts, uint64_t(B) * 4, false);
  ranges[nr++] = range(d_flags, 4, true);
  if (written_overlap(ranges, nr)) return SWRT_E_INVALID_ARG;
  const int vec = align_acc % 16 == 0 ? 16 : align_acc % 8 == 0 ? 8 : align_acc % 4 == 0 ? 4
                : align_acc % 2 == 0 ? 2 : 1;
  const int64_t row_words = row / vec;
  if (!mul_ok(C + S, row_words, &t) || t >= (int64_t(1) << 31) - kBlock * kUnroll)
    return SWRT_E_UNSUPPORTED;
  {
    const uint64_t tile_words = kBlock * kUnroll;
    const uint64_t tiles = (uint64_t(C + S) * row_words + tile_words - 1) / tile_words;
    if (S > 1 && uint64_t(slices) * tiles >= (uint64_t(1) << 31)) return SWRT_E_UNSUPPORTED;
  }

  a.lp = cache_past_lens;
  a.ev = evict_counts;
  a.flags = d_flags;
  a.nb_b = nb[0];
  a.nb_h = nb[1];
  a.nb_s = nb[2];
  a.row_bytes = uint64_t(row);
  a.H = uint32_t(H);
  a.BH = uint32_t(B * H);
  a.tiles = 1;
  a.row_words = uint32_t(row_words);
  a.C = capacity;
  a.S = seq_len;
  a.by_row = FastDiv(uint32_t(row_words));

  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint32_t ns = uint32_t(slices);
  if (n_layers == 1) {
    WinArgs<1> one;
    one.cache[0][0] = a.cache[0][0];
    one.cache[0][1] = a.cache[0][1];
    one.nw[0][0] = a.nw[0][0];
    one.nw[0][1] = a.nw[0][1];
    one.stage[0][0] = a.stage[0][0];
    one.stage[0][1] = a.stage[0][1];
    one.lp = a.lp;
    one.ev = a.ev;
    one.flags = a.flags;
    one.nb_b = a.nb_b;
    one.nb_h = a.nb_h;
    one.nb_s = a.nb_s;
    one.row_bytes = a.row_bytes;
    one.H = a.H;
    one.BH = a.BH;
    one.tiles = a.tiles;
    one.row_words = a.row_words;
    one.C = a.C;
    one.S = a.S;
    one.by_row = a.by_row;
    switch (vec) {
      case 16: return launch<16>(one, ns, phase, st);
      case 8: return launch<8>(one, ns, phase, st);
      case 4: return launch<4>(one, ns, phase, st);
      case 2: return launch<2>(one, ns, phase, st);
      default: return launch<1>(one, ns, phase, st);
    }
  }
  switch (vec) {
    case 16: return launch<16>(a, ns, phase, st);
    case 8: return launch<8>(a, ns, phase, st);
    case 4: return launch<4>(a, ns, phase, st);
    case 2: return launch<2>(a, ns, phase, st);
    default: return launch<1>(a, ns, phase, st);
  }
}

}  // namespace
}  // namespace swrt

extern "C" int swrt_kv_window_append(void *k_cache, void *v_cache, const void *k_new,
                                     const void *v_new, const int64_t *new_strides,
                                     void *k_staging, void *v_staging,
                                     const int32_t *cache_past_lens, const int32_t *evict_counts,
                                     int batch, int kv_heads, int capacity, int seq_len,
                                     int head_dim, int elem_bits, unsigned phase,
                                     uint32_t *d_flags, void *stream) {
  return swrt::window_append(1, &k_cache, &v_cache, &k_new, &v_new, new_strides, &k_staging,
                             &v_staging, cache_past_lens, evict_counts, batch, kv_heads, capacity,
                             seq_len, head_dim, elem_bits, phase, d_flags, stream);
}

extern "C" int swrt_kv_window_append_layers(int n_layers, void *const *k_caches,
                                            void *const *v_caches, const void *const *k_news,
                                            const void *const *v_news, const int64_t *new_strides,
                                            void *const *k_stagings, void *const *v_stagings,
                                            const int32_t *cache_past_lens,
                                            const int32_t *evict_counts, int batch, int kv_heads,
                                            int capacity, int seq_len, int head_dim, int elem_bits,
                                            unsigned phase, uint32_t *d_flags, void *stream) {
  return swrt::window_append(n_layers, k_caches, v_caches, k_news, v_news, new_strides, k_stagings,
                             v_stagings, cache_past_lens, evict_counts, batch, kv_heads, capacity,
                             seq_len, head_dim, elem_bits, phase, d_flags, stream);
}
