// kv_window.hip -- the windowed GQA cache step on gfx950 (onnxruntime pull
// request "GQA support sliding_window_cache", section "Design"; the device
// bodies and their ordering argument are in window_device.hpp).
//
// Kernels (K and V of every layer in the same launch; one slice = one
// (layer, tensor, b, h); consecutive workgroups walk consecutive slices):
//   window_in_place  S = 1: one workgroup per slice, shift by E then append.
//   window_stage     S > 1, phase STAGE: 16 KiB tiles of each staging slice.
//   window_commit    S > 1, phase COMMIT: 16 KiB tiles of each cache slice.
//   window_stage_lengths
//                    the lengths of the step and phase STAGE in one launch
//                    (swrt_kv_window_stage_step).
// Batch entries whose (Lp, E) pair is not a step that fits (C, S) are flagged
// and left untouched. The XF instances are the fused append (xf_device.hpp):
// new rows pass through the row transform at positions past_lens[b] + s, and
// entries whose positions leave the rotary tables are flagged and skipped.
#include "swrt_host.hpp"

namespace swrt {
namespace {

template <int NL>
struct WinArgs {
  char *cache[NL][2];
  const char *nw[NL][2];
  char *stage[NL][2];
  WindowGeom g;
  RowXf xf;  // fused append only
};

template <int VEC, int NL, int SPW, bool XF>
__global__ __launch_bounds__(kWinBlock) void window_in_place(WinArgs<NL> a) {
  if constexpr (SPW == 1) {
    const Slice s = decode_slice(a.g, blockIdx.x);
    const int64_t Lp = ld_invariant(a.g.lp, s.b), E = ld_invariant(a.g.ev, s.b);
    if (!lengths_ok(a.g, s, threadIdx.x == 0, Lp, E)) return;
    int64_t P = 0;
    if constexpr (XF) {
      P = a.g.past[s.b];
      if (!positions_ok(a.g, a.xf, s, threadIdx.x == 0, P)) return;
    }
    char *base = a.cache[s.layer][s.t] + uint64_t(s.b * a.g.H + s.h) * uint64_t(a.g.C) * a.g.row_bytes;
    shift_append_slice<VEC, kWinBlock, kWinUnroll, XF>(
        base, a.nw[s.layer][s.t] + s.b * a.g.nb_b + s.h * a.g.nb_h, Lp, E, a.g.row_bytes,
        a.g.row_words, &a.xf, int(s.t), P, s.h);
  } else {
    constexpr uint32_t GB = kWinBlock / SPW;
    shift_append_group<VEC, SPW, XF>(
        blockIdx.x * SPW, a.g.slices, a.g.row_bytes, a.g.row_words,
        [&](uint32_t slice, int g) {
          const Slice s = decode_slice(a.g, slice);
          SliceWork w;
          w.Lp = ld_invariant(a.g.lp, s.b);
          w.E = ld_invariant(a.g.ev, s.b);
          w.ok = lengths_ok(a.g, s, threadIdx.x == g * GB, w.Lp, w.E);
          w.t = int(s.t);
          w.h = s.h;
          w.pos = 0;
          if constexpr (XF) {
            w.pos = a.g.past[s.b];
            w.ok = w.ok && positions_ok(a.g, a.xf, s, threadIdx.x == g * GB, w.pos);
          }
          w.base = a.cache[s.layer][s.t] + uint64_t(s.b * a.g.H + s.h) * uint64_t(a.g.C) * a.g.row_bytes;
          w.new_row = a.nw[s.layer][s.t] + s.b * a.g.nb_b + s.h * a.g.nb_h;
          return w;
        },
        &a.xf);
  }
}

template <int VEC, int NL, bool XF>
__global__ __launch_bounds__(kWinBlock) void window_stage(WinArgs<NL> a) {
  const uint32_t slice = blockIdx.x / a.g.tiles, tile = blockIdx.x - slice * a.g.tiles;
  const Slice s = decode_slice(a.g, slice);
  const int64_t Lp = ld_invariant(a.g.lp, s.b), E = ld_invariant(a.g.ev, s.b);
  if (!lengths_ok(a.g, s, tile == 0 && threadIdx.x == 0, Lp, E)) return;
  int64_t P = 0;
  if constexpr (XF) {
    P = a.g.past[s.b];
    if (!positions_ok(a.g, a.xf, s, tile == 0 && threadIdx.x == 0, P)) return;
  }
  const uint64_t bh = s.b * a.g.H + s.h;
  stage_tile<VEC, XF>(a.g, a.cache[s.layer][s.t] + bh * uint64_t(a.g.C) * a.g.row_bytes,
                      a.stage[s.layer][s.t] + bh * uint64_t(a.g.C + a.g.S) * a.g.row_bytes,
                      a.nw[s.layer][s.t] + s.b * a.g.nb_b + s.h * a.g.nb_h, Lp, tile, &a.xf,
                      int(s.t), P, s.h);
}

template <int VEC, int NL, bool XF>
__global__ __launch_bounds__(kWinBlock) void window_commit(WinArgs<NL> a) {
  const uint32_t slice = blockIdx.x / a.g.tiles, tile = blockIdx.x - slice * a.g.tiles;
  const Slice s = decode_slice(a.g, slice);
  const int64_t Lp = ld_invariant(a.g.lp, s.b), E = ld_invariant(a.g.ev, s.b);
  if (!lengths_ok(a.g, s, tile == 0 && threadIdx.x == 0, Lp, E)) return;
  if constexpr (XF) {  // an entry the stage phase skipped stays untouched
    if (!positions_ok(a.g, a.xf, s, tile == 0 && threadIdx.x == 0, a.g.past[s.b])) return;
  }
  const uint64_t bh = s.b * a.g.H + s.h;
  commit_tile<VEC>(a.g, a.cache[s.layer][s.t] + bh * uint64_t(a.g.C) * a.g.row_bytes,
                   a.stage[s.layer][s.t] + bh * uint64_t(a.g.C + a.g.S) * a.g.row_bytes, Lp, E,
                   tile);
}

// The lengths of a staged step and its STAGE phase in one grid. The first
// len_blocks workgroups (one batch entry per thread) write the length arrays
// with the arithmetic of kv_seq_lengths; every stage workgroup derives its
// slice's Lp from seqlens_k the same way, so its pair is always one the step
// accepts. The COMMIT launch that follows reads the written arrays. The XF
// instances transform the new rows at positions P + s, P derived alike.
struct StageLengths {
  const int32_t *seqlens_k;
  int64_t *total, *past;
  int32_t *cache_past, *cache_total, *evict;
  FastDiv gap;  // capacity - window + 1
  int32_t batch;
  uint32_t len_blocks, stage_blocks;
};

template <int VEC, int NL, bool DRIFT, bool XF>
__global__ __launch_bounds__(kWinBlock) void window_stage_lengths(WinArgs<NL> a, StageLengths q) {
  const uint32_t bid = blockIdx.x;
  if (bid < q.len_blocks) {  // no barrier in this part
    const int32_t b = int32_t(bid * kWinBlock + threadIdx.x);
    if (b < q.batch) {
      const StepLengths r = step_lengths<DRIFT>(q.seqlens_k[b], a.g.S, a.g.C, q.gap);
      if (r.bad && a.g.flags) atomicOr(a.g.flags, SWRT_FLAG_BAD_SEQLEN);
      if (q.total) q.total[b] = r.T;
      if (q.past) q.past[b] = r.P;
      q.cache_past[b] = int32_t(r.Lp);
      if (q.cache_total) q.cache_total[b] = int32_t(r.L);
      q.evict[b] = int32_t(r.E);
    }
  }
  if (bid >= q.stage_blocks) return;  // a grid sized by the length arrays alone
  const uint32_t slice = bid / a.g.tiles, tile = bid - slice * a.g.tiles;
  const Slice s = decode_slice(a.g, slice);
  const StepLengths r = step_lengths<DRIFT>(ld_invariant(q.seqlens_k, s.b), a.g.S, a.g.C, q.gap);
  if constexpr (XF) {
    if (!positions_ok(a.g, a.xf, s, tile == 0 && threadIdx.x == 0, r.P)) return;
  }
  const uint64_t bh = s.b * a.g.H + s.h;
  stage_tile<VEC, XF>(a.g, a.cache[s.layer][s.t] + bh * uint64_t(a.g.C) * a.g.row_bytes,
                      a.stage[s.layer][s.t] + bh * uint64_t(a.g.C + a.g.S) * a.g.row_bytes,
                      a.nw[s.layer][s.t] + s.b * a.g.nb_b + s.h * a.g.nb_h, r.Lp, tile, &a.xf,
                      int(s.t), r.P, s.h);
}

template <int VEC, int NL, bool XF>
int launch(const WindowPlan &p, unsigned phase, hipStream_t stream) {
  WinArgs<NL> a;
  for (int l = 0; l < NL && l < p.n_layers; ++l)
    for (int t = 0; t < 2; ++t) {
      a.cache[l][t] = p.cache[l][t];
      a.nw[l][t] = p.nw[l][t];
      a.stage[l][t] = p.stage[l][t];
    }
  a.g = p.g;
  a.xf = p.xf;
  if (p.g.S == 1) {
    const int spw = slices_per_group(p.g.C, p.g.row_words, XF,
                                     XF ? int64_t(p.g.row_bytes / uint64_t(p.xf.out_bytes)) : 0);
    const dim3 grid((p.slices + spw - 1) / spw);
    if (spw == 4)
      hipLaunchKernelGGL((window_in_place<VEC, NL, 4, XF>), grid, dim3(kWinBlock), 0, stream, a);
    else if (spw == 2)
      hipLaunchKernelGGL((window_in_place<VEC, NL, 2, XF>), grid, dim3(kWinBlock), 0, stream, a);
    else
      hipLaunchKernelGGL((window_in_place<VEC, NL, 1, XF>), grid, dim3(kWinBlock), 0, stream, a);
    return launch_status();
  }
  if (phase & SWRT_PHASE_STAGE) {
    a.g.tiles = uint32_t((uint64_t(p.g.C + p.g.S) * p.g.row_words + kWinTile - 1) / kWinTile);
    hipLaunchKernelGGL((window_stage<VEC, NL, XF>), dim3(p.slices * a.g.tiles), dim3(kWinBlock), 0,
                       stream, a);
    if (launch_status() != SWRT_OK) return SWRT_E_LAUNCH;
  }
  if (phase & SWRT_PHASE_COMMIT) {
    a.g.tiles = uint32_t((uint64_t(p.g.C) * p.g.row_words + kWinTile - 1) / kWinTile);
    hipLaunchKernelGGL((window_commit<VEC, NL, XF>), dim3(p.slices * a.g.tiles), dim3(kWinBlock), 0,
                       stream, a);
    if (launch_status() != SWRT_OK) return SWRT_E_LAUNCH;
  }
  return SWRT_OK;
}

template <int NL, bool XF>
int dispatch(const WindowPlan &p, int vec, unsigned phase, hipStream_t s) {
  switch (vec) {
    case 16: return launch<16, NL, XF>(p, phase, s);
    case 8: return launch<8, NL, XF>(p, phase, s);
    case 4: return launch<4, NL, XF>(p, phase, s);
    case 2: return launch<2, NL, XF>(p, phase, s);
    default: return launch<1, NL, XF>(p, phase, s);
  }
}

template <int VEC, int NL, bool XF>
int launch_stage_lengths(const WindowPlan &p, const StageLengths &q, bool drift, uint32_t grid,
                         hipStream_t stream) {
  WinArgs<NL> a;
  for (int l = 0; l < NL && l < p.n_layers && !p.empty; ++l)
    for (int t = 0; t < 2; ++t) {
      a.cache[l][t] = p.cache[l][t];
      a.nw[l][t] = p.nw[l][t];
      a.stage[l][t] = p.stage[l][t];
    }
  a.g = p.g;
  a.xf = p.xf;
  if (drift)
    hipLaunchKernelGGL((window_stage_lengths<VEC, NL, true, XF>), dim3(grid), dim3(kWinBlock), 0,
                       stream, a, q);
  else
    hipLaunchKernelGGL((window_stage_lengths<VEC, NL, false, XF>), dim3(grid), dim3(kWinBlock),
                       0, stream, a, q);
  return launch_status();
}

template <int NL, bool XF>
int dispatch_stage_lengths(const WindowPlan &p, const StageLengths &q, int vec, bool drift,
                           uint32_t grid, hipStream_t s) {
  switch (vec) {
    case 16: return launch_stage_lengths<16, NL, XF>(p, q, drift, grid, s);
    case 8: return launch_stage_lengths<8, NL, XF>(p, q, drift, grid, s);
    case 4: return launch_stage_lengths<4, NL, XF>(p, q, drift, grid, s);
    case 2: return launch_stage_lengths<2, NL, XF>(p, q, drift, grid, s);
    default: return launch_stage_lengths<1, NL, XF>(p, q, drift, grid, s);
  }
}

// the lengths (kv_seq_lengths_drift with this window) and phase STAGE of
// swrt_kv_window_append_layers (xf: of swrt_kv_window_append_xf) in one launch
int stage_step(int n_layers, void *const *k_caches, void *const *v_caches,
               const void *const *k_news, const void *const *v_news, const int64_t *new_strides,
               void *const *k_stagings, void *const *v_stagings, const int32_t *seqlens_k,
               int capacity, int window, int64_t *total_lens, int64_t *past_lens,
               int32_t *cache_past_lens, int32_t *cache_total_lens, int32_t *evict_counts,
               int batch, int kv_heads, int seq_len, int head_dim, int elem_bits,
               const swrt_row_transform *xf, uint32_t *d_flags, void *stream) {
  if (batch < 0 || capacity < 1 || seq_len < 2) return SWRT_E_INVALID_ARG;
  if (window < 1 || window > capacity) return SWRT_E_INVALID_ARG;
  WindowPlan p{};
  Range ranges[6 * kMaxLayers + 20];
  int nr = 0;
  RowXf x{};
  int st;
  if (xf) {
    if ((st = plan_xf(xf, head_dim, kv_heads, &x, ranges, &nr)) != SWRT_OK) return st;
    elem_bits = x.out_bytes * 8;
  }
  st = plan_window(n_layers, k_caches, v_caches, k_news, v_news, new_strides, k_stagings,
                   v_stagings, nullptr, nullptr, true, batch, kv_heads, capacity, seq_len,
                   head_dim, elem_bits, SWRT_PHASE_STAGE, d_flags, xf ? &x : nullptr, &p, ranges,
                   &nr);
  if (st != SWRT_OK) return st;
  // the commit reads Lp and E (and, fused, P): those arrays are required
  if (batch > 0 && (!seqlens_k || !cache_past_lens || !evict_counts || (xf && !past_lens)))
    return SWRT_E_INVALID_ARG;
  if (addr_of(seqlens_k) % 4 || addr_of(total_lens) % 8 || addr_of(past_lens) % 8 ||
      addr_of(cache_past_lens) % 4 || addr_of(cache_total_lens) % 4 || addr_of(evict_counts) % 4 ||
      addr_of(d_flags) % 4)
    return SWRT_E_INVALID_ARG;
  const uint64_t B = uint64_t(batch);
  ranges[nr++] = range(seqlens_k, B * 4, false);
  ranges[nr++] = range(total_lens, B * 8, true);
  ranges[nr++] = range(past_lens, B * 8, true);
  ranges[nr++] = range(cache_past_lens, B * 4, true);
  ranges[nr++] = range(cache_total_lens, B * 4, true);
  ranges[nr++] = range(evict_counts, B * 4, true);
  ranges[nr++] = range(d_flags, 4, true);
  if (written_overlap(ranges, nr)) return SWRT_E_INVALID_ARG;
  if (batch == 0) return SWRT_OK;
  const int vec = p.empty ? 16 : word_of(p.align);
  if (!p.empty && (st = finish_window(&p, vec)) != SWRT_OK) return st;
  uint64_t tiles = 1, stage_blocks = 0;
  if (!p.empty) {
    tiles = (uint64_t(capacity + seq_len) * p.g.row_words + kWinTile - 1) / kWinTile;
    stage_blocks = uint64_t(p.slices) * tiles;
  }
  p.g.tiles = uint32_t(tiles);
  p.g.C = capacity;
  p.g.S = seq_len;
  p.g.flags = d_flags;
  StageLengths q{seqlens_k, total_lens, past_lens, cache_past_lens, cache_total_lens, evict_counts,
                 FastDiv(uint32_t(capacity - window + 1)), batch,
                 uint32_t((B + kWinBlock - 1) / kWinBlock), uint32_t(stage_blocks)};
  const uint64_t grid = stage_blocks > q.len_blocks ? stage_blocks : q.len_blocks;
  if (grid >= (uint64_t(1) << 31)) return SWRT_E_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool drift = window < capacity;
  if (xf)
    return n_layers <= 1 ? dispatch_stage_lengths<1, true>(p, q, vec, drift, uint32_t(grid), s)
                         : dispatch_stage_lengths<kMaxLayers, true>(p, q, vec, drift,
                                                                    uint32_t(grid), s);
  return n_layers <= 1 ? dispatch_stage_lengths<1, false>(p, q, vec, drift, uint32_t(grid), s)
                       : dispatch_stage_lengths<kMaxLayers, false>(p, q, vec, drift,
                                                                   uint32_t(grid), s);
}

// xf: the fused append's transform (null: a plain copy), with past_lens
int window_append(int n_layers, void *const *k_caches, void *const *v_caches,
                  const void *const *k_news, const void *const *v_news,
                  const int64_t *new_strides, void *const *k_stagings, void *const *v_stagings,
                  const int32_t *cache_past_lens, const int32_t *evict_counts, int batch,
                  int kv_heads, int capacity, int seq_len, int head_dim, int elem_bits,
                  unsigned phase, const swrt_row_transform *xf, const int64_t *past_lens,
                  uint32_t *d_flags, void *stream) {
  WindowPlan p;
  Range ranges[6 * kMaxLayers + 16];
  int nr = 0;
  RowXf x{};
  int st;
  if (xf) {
    if ((st = plan_xf(xf, head_dim, kv_heads, &x, ranges, &nr)) != SWRT_OK) return st;
    elem_bits = x.out_bytes * 8;
    // in place, the appended row is spread over one workgroup's lanes
    if (seq_len == 1 && head_dim > kXfLaneElems * kWinBlock) return SWRT_E_UNSUPPORTED;
  }
  st = plan_window(n_layers, k_caches, v_caches, k_news, v_news, new_strides, k_stagings,
                   v_stagings, cache_past_lens, evict_counts, false, batch, kv_heads, capacity,
                   seq_len, head_dim, elem_bits, phase, d_flags, xf ? &x : nullptr, &p, ranges,
                   &nr);
  if (st != SWRT_OK || p.empty) return st;
  if (xf) {
    if (!past_lens || addr_of(past_lens) % 8) return SWRT_E_INVALID_ARG;
    ranges[nr++] = range(past_lens, uint64_t(batch) * 8, false);
    p.g.past = past_lens;
  }
  ranges[nr++] = range(d_flags, 4, true);
  if (written_overlap(ranges, nr)) return SWRT_E_INVALID_ARG;
  const int vec = word_of(p.align);
  if ((st = finish_window(&p, vec)) != SWRT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (xf)
    return n_layers == 1 ? dispatch<1, true>(p, vec, phase, s)
                         : dispatch<kMaxLayers, true>(p, vec, phase, s);
  return n_layers == 1 ? dispatch<1, false>(p, vec, phase, s)
                       : dispatch<kMaxLayers, false>(p, vec, phase, s);
}

}  // namespace

// ---------------------------------------------------------------------------
// plans (declared in swrt_host.hpp)
// ---------------------------------------------------------------------------
int plan_window(int n_layers, void *const *k_caches, void *const *v_caches,
                const void *const *k_news, const void *const *v_news, const int64_t *new_strides,
                void *const *k_stagings, void *const *v_stagings, const int32_t *cache_past_lens,
                const int32_t *evict_counts, bool lengths_in_kernel, int batch, int kv_heads,
                int capacity, int seq_len, int head_dim, int elem_bits, unsigned phase,
                uint32_t *d_flags, const RowXf *xf, WindowPlan *p, Range *ranges, int *nr) {
  p->empty = true;
  p->xf = xf ? *xf : RowXf{};
  p->g.past = nullptr;
  p->n_layers = n_layers;
  if (n_layers < 0 || n_layers > kMaxLayers) return SWRT_E_INVALID_ARG;
  if (batch < 0 || kv_heads < 0 || head_dim < 0 || capacity < 1 || seq_len < 1)
    return SWRT_E_INVALID_ARG;
  if (!valid_elem_bits(elem_bits)) return SWRT_E_INVALID_ARG;
  const int64_t B = batch, H = kv_heads, C = capacity, S = seq_len, D = head_dim;
  if (S > 1 && phase != SWRT_PHASE_STAGE && phase != SWRT_PHASE_COMMIT && phase != SWRT_PHASE_ALL)
    return SWRT_E_INVALID_ARG;
  if (!new_strides) return SWRT_E_INVALID_ARG;
  if ((D * elem_bits) % 8) return SWRT_E_UNSUPPORTED;
  // new rows: the cache's elements, or the fused append's input elements
  const int new_bits = xf ? xf->in_bytes * 8 : elem_bits;
  int64_t nb[3];
  for (int i = 0; i < 3; ++i) {
    if (new_strides[i] < 0) return SWRT_E_INVALID_ARG;
    if (!mul_ok(new_strides[i], new_bits, &nb[i]) || nb[i] % 8) return SWRT_E_UNSUPPORTED;
    nb[i] /= 8;
  }
  const int64_t row = D * elem_bits / 8;
  const int64_t new_row = D * new_bits / 8;
  p->row = row;
  if (n_layers == 0 || B == 0 || H == 0 || row == 0) return SWRT_OK;
  if (!k_caches || !v_caches || !k_news || !v_news) return SWRT_E_INVALID_ARG;
  if (!lengths_in_kernel && (!cache_past_lens || !evict_counts)) return SWRT_E_INVALID_ARG;
  if (S > 1 && (!k_stagings || !v_stagings)) return SWRT_E_INVALID_ARG;

  // B, H, C, S < 2^31: B * H and C + S fit; every later product is checked
  int64_t slices, bhc, bhcs, cache_bytes, stage_bytes;
  if (!mul_ok(B * H, 2 * int64_t(n_layers), &slices) || slices >= (int64_t(1) << 31))
    return SWRT_E_UNSUPPORTED;
  if (!mul_ok(B * H, C, &bhc) || !mul_ok(B * H, C + S, &bhcs) ||
      !mul_ok(bhc, row, &cache_bytes) || !mul_ok(bhcs, row, &stage_bytes))
    return SWRT_E_UNSUPPORTED;
  int64_t new_span = new_row;  // the last new row's end: (B-1, H-1, S-1) strides on
  const int64_t last[3] = {B - 1, H - 1, S - 1};
  for (int i = 0; i < 3; ++i) {
    int64_t t;
    if (!mul_ok(last[i], nb[i], &t) || __builtin_add_overflow(new_span, t, &new_span))
      return SWRT_E_UNSUPPORTED;
  }
  const uint64_t align = elem_align(elem_bits), new_align = elem_align(new_bits);
  if (addr_of(cache_past_lens) % 4 || addr_of(evict_counts) % 4 || addr_of(d_flags) % 4)
    return SWRT_E_INVALID_ARG;

  // the copy word must divide every copied address and stride; fused-append
  // new rows are read element by element, so they do not count
  uint64_t acc = uint64_t(row) | (xf ? 0 : uint64_t(nb[0]) | uint64_t(nb[1]) | uint64_t(nb[2]));
  // caches and staging buffers are written: nothing may overlap them (across
  // layers too); new rows and lengths are only read and may be shared
  for (int l = 0; l < n_layers; ++l) {
    const void *q[6] = {k_caches[l], v_caches[l], k_news[l], v_news[l],
                        S > 1 ? k_stagings[l] : nullptr, S > 1 ? v_stagings[l] : nullptr};
    const uint64_t n[6] = {uint64_t(cache_bytes), uint64_t(cache_bytes), uint64_t(new_span),
                           uint64_t(new_span), uint64_t(stage_bytes), uint64_t(stage_bytes)};
    for (int i = 0; i < (S > 1 ? 6 : 4); ++i) {
      const bool is_new = i == 2 || i == 3;
      if (!q[i] || addr_of(q[i]) % (is_new ? new_align : align)) return SWRT_E_INVALID_ARG;
      if (!(xf && is_new)) acc |= addr_of(q[i]);
      ranges[(*nr)++] = range(q[i], n[i], !is_new);
    }
    p->cache[l][0] = static_cast<char *>(k_caches[l]);
    p->cache[l][1] = static_cast<char *>(v_caches[l]);
    p->nw[l][0] = static_cast<const char *>(k_news[l]);
    p->nw[l][1] = static_cast<const char *>(v_news[l]);
    p->stage[l][0] = S > 1 ? static_cast<char *>(k_stagings[l]) : nullptr;
    p->stage[l][1] = S > 1 ? static_cast<char *>(v_stagings[l]) : nullptr;
  }
  if (!lengths_in_kernel) {
    ranges[(*nr)++] = range(cache_past_lens, uint64_t(B) * 4, false);
    ranges[(*nr)++] = range(evict_counts, uint64_t(B) * 4, false);
  }
  p->align = acc;
  p->slices = uint32_t(slices);
  p->g.slices = uint32_t(slices);
  p->g.lp = lengths_in_kernel ? nullptr : cache_past_lens;
  p->g.ev = lengths_in_kernel ? nullptr : evict_counts;
  p->g.flags = d_flags;
  p->g.nb_b = nb[0];
  p->g.nb_h = nb[1];
  p->g.nb_s = nb[2];
  p->g.row_bytes = uint64_t(row);
  p->g.H = uint32_t(H);
  p->g.BH = uint32_t(B * H);
  p->g.tiles = 1;
  p->g.C = capacity;
  p->g.S = seq_len;
  p->empty = false;
  return SWRT_OK;
}

int finish_window(WindowPlan *p, int vec) {
  const int64_t row_words = p->row / vec, C = p->g.C, S = p->g.S;
  int64_t t;
  if (!mul_ok(C + S, row_words, &t) || t >= (int64_t(1) << 31) - kWinTile)
    return SWRT_E_UNSUPPORTED;
  const uint64_t tiles = (uint64_t(C + S) * row_words + kWinTile - 1) / kWinTile;
  if (S > 1 && uint64_t(p->slices) * tiles >= (uint64_t(1) << 31)) return SWRT_E_UNSUPPORTED;
  p->g.row_words = uint32_t(row_words);
  p->g.by_row = FastDiv(uint32_t(row_words));
  return SWRT_OK;
}

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
                             seq_len, head_dim, elem_bits, phase, nullptr, nullptr, d_flags,
                             stream);
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
                             seq_len, head_dim, elem_bits, phase, nullptr, nullptr, d_flags,
                             stream);
}

extern "C" int swrt_kv_window_append_xf(int n_layers, void *const *k_caches,
                                        void *const *v_caches, const void *const *k_news,
                                        const void *const *v_news, const int64_t *new_strides,
                                        void *const *k_stagings, void *const *v_stagings,
                                        const int32_t *cache_past_lens,
                                        const int32_t *evict_counts, const int64_t *past_lens,
                                        int batch, int kv_heads, int capacity, int seq_len,
                                        int head_dim, unsigned phase,
                                        const swrt_row_transform *xf, uint32_t *d_flags,
                                        void *stream) {
  if (!xf) return SWRT_E_INVALID_ARG;
  return swrt::window_append(n_layers, k_caches, v_caches, k_news, v_news, new_strides, k_stagings,
                             v_stagings, cache_past_lens, evict_counts, batch, kv_heads, capacity,
                             seq_len, head_dim, 8, phase, xf, past_lens, d_flags, stream);
}

extern "C" int swrt_kv_window_stage_step(int n_layers, void *const *k_caches,
                                         void *const *v_caches, const void *const *k_news,
                                         const void *const *v_news, const int64_t *new_strides,
                                         void *const *k_stagings, void *const *v_stagings,
                                         const int32_t *seqlens_k, int capacity, int window,
                                         int64_t *total_lens, int64_t *past_lens,
                                         int32_t *cache_past_lens, int32_t *cache_total_lens,
                                         int32_t *evict_counts, int batch, int kv_heads,
                                         int seq_len, int head_dim, int elem_bits,
                                         uint32_t *d_flags, void *stream) {
  return swrt::stage_step(n_layers, k_caches, v_caches, k_news, v_news, new_strides, k_stagings,
                          v_stagings, seqlens_k, capacity, window, total_lens, past_lens,
                          cache_past_lens, cache_total_lens, evict_counts, batch, kv_heads,
                          seq_len, head_dim, elem_bits, nullptr, d_flags, stream);
}

extern "C" int swrt_kv_window_stage_step_xf(
    int n_layers, void *const *k_caches, void *const *v_caches, const void *const *k_news,
    const void *const *v_news, const int64_t *new_strides, void *const *k_stagings,
    void *const *v_stagings, const int32_t *seqlens_k, int capacity, int window,
    int64_t *total_lens, int64_t *past_lens, int32_t *cache_past_lens, int32_t *cache_total_lens,
    int32_t *evict_counts, int batch, int kv_heads, int seq_len, int head_dim,
    const swrt_row_transform *xf, uint32_t *d_flags, void *stream) {
  if (!xf) return SWRT_E_INVALID_ARG;
  return swrt::stage_step(n_layers, k_caches, v_caches, k_news, v_news, new_strides, k_stagings,
                          v_stagings, seqlens_k, capacity, window, total_lens, past_lens,
                          cache_past_lens, cache_total_lens, evict_counts, batch, kv_heads,
                          seq_len, head_dim, 8, xf, d_flags, stream);
}
