// tensor_scatter.hip -- ONNX TensorScatter on gfx950 (operator page
// "TensorScatter", ai.onnx since version 24; the device bodies are in
// scatter_device.hpp).
//
// In place (present == past) only the O*S target rows move: one thread per
// raw-bit word of the update, consecutive threads on consecutive words, so the
// update is read and the target rows are written fully coalesced. Out of place
// every present row is produced in one pass from either past or the update.
// A batched call runs every tensor of one shape in a single grid. The XF
// instances are the fused append (row transform on the update rows).
#include "swrt_host.hpp"

namespace swrt {
namespace {

template <int NT>
struct ScatterArgs {
  char *present[NT];
  const char *past[NT];
  const char *update[NT];
  uint32_t tiles;  // tiles per tensor
  ScatterGeom g;
  RowXf xf;        // fused append only
  uint64_t vmask;  // fused append: bit t set when tensor t is a V cache
};

constexpr uint32_t kTile = kScatBlock * kScatUnroll;

template <int VEC, int NT, bool XF>
__global__ __launch_bounds__(kScatBlock) void scatter_in_place(ScatterArgs<NT> a) {
  __shared__ TileBatches<kTile, XF> tb;
  const uint32_t t = blockIdx.x / a.tiles;  // which tensor of a batched call
  const uint32_t tile = (blockIdx.x - t * a.tiles) * kTile;
  scatter_in_place_tile<VEC, kScatBlock, XF>(a.g, a.present[t], a.update[t], tile, tb, &a.xf,
                                             int((a.vmask >> t) & 1));
}

template <int VEC, int NT, bool XF>
__global__ __launch_bounds__(kScatBlock) void scatter_out_of_place(ScatterArgs<NT> a) {
  __shared__ TileBatches<kTile, XF> tb;
  const uint32_t t = blockIdx.x / a.tiles;
  const uint32_t tile = (blockIdx.x - t * a.tiles) * kTile;
  scatter_out_of_place_tile<VEC, kScatBlock, XF>(a.g, a.present[t], a.past[t], a.update[t], tile,
                                                 tb, &a.xf, int((a.vmask >> t) & 1));
}

template <int VEC, int NT, bool XF>
int launch(const ScatterPlan &p, uint64_t vmask, hipStream_t stream) {
  ScatterArgs<NT> a;
  for (int t = 0; t < NT && t < p.n; ++t) {
    a.present[t] = p.present[t];
    a.past[t] = p.past[t];
    a.update[t] = p.update[t];
  }
  a.tiles = p.tiles;
  a.g = p.g;
  a.xf = p.xf;
  a.vmask = vmask;
  const dim3 grid(p.tiles * uint32_t(p.n));
  if (p.in_place)
    hipLaunchKernelGGL((scatter_in_place<VEC, NT, XF>), grid, dim3(kScatBlock), 0, stream, a);
  else
    hipLaunchKernelGGL((scatter_out_of_place<VEC, NT, XF>), grid, dim3(kScatBlock), 0, stream, a);
  return launch_status();
}

template <int NT, bool XF>
int dispatch(const ScatterPlan &p, int vec, uint64_t vmask, hipStream_t s) {
  switch (vec) {
    case 16: return launch<16, NT, XF>(p, vmask, s);
    case 8: return launch<8, NT, XF>(p, vmask, s);
    case 4: return launch<4, NT, XF>(p, vmask, s);
    case 2: return launch<2, NT, XF>(p, vmask, s);
    default: return launch<1, NT, XF>(p, vmask, s);
  }
}

// xf: the fused append's transform (null: a plain copy); tensors: K (0) or V
// (1) per tensor, with xf
int scatter(int n_tensors, void *const *presents, const void *const *pasts,
            const void *const *updates, const int64_t *write_indices, const int64_t *shape,
            int rank, int axis, int64_t seq_len, int mode, int elem_bits,
            const swrt_row_transform *xf, const int *tensors, uint32_t *d_flags, void *stream) {
  ScatterPlan p;
  Range ranges[3 * kMaxTensors + 13];
  int nr = 0;
  RowXf x{};
  uint64_t vmask = 0;
  int st;
  if (n_tensors < 0 || n_tensors > kMaxTensors) return SWRT_E_INVALID_ARG;  // before any array
  if (xf) {
    if (!shape || rank < 3 || rank > SWRT_MAX_RANK) return SWRT_E_INVALID_ARG;
    // per-channel tables: [shape[1], head_dim] of a [B, H, M, D] cache, one row for rank 3
    if (rank > 4 && (xf->channel_scale[0] || xf->channel_scale[1] || xf->channel_zero_point[0] ||
                     xf->channel_zero_point[1]))
      return SWRT_E_INVALID_ARG;
    if ((st = plan_xf(xf, shape[rank - 1], rank == 4 ? shape[1] : 1, &x, ranges, &nr)) != SWRT_OK)
      return st;
    if (n_tensors > 0 && !tensors) return SWRT_E_INVALID_ARG;
    for (int t = 0; t < n_tensors; ++t) {
      if (tensors[t] != 0 && tensors[t] != 1) return SWRT_E_INVALID_ARG;
      vmask |= uint64_t(tensors[t]) << t;
    }
    elem_bits = x.out_bytes * 8;
  }
  st = plan_scatter(n_tensors, presents, pasts, updates, write_indices, shape, rank, axis,
                    seq_len, mode, elem_bits, d_flags, xf ? &x : nullptr, &p, ranges, &nr);
  if (st != SWRT_OK) return st;
  ranges[nr++] = range(d_flags, 4, true);
  if (written_overlap(ranges, nr)) return SWRT_E_INVALID_ARG;
  if (p.empty) return SWRT_OK;
  int vec = word_of(p.align);
  if (xf && vec > 4) vec = 4;  // fused append: few elements to transform per lane
  if ((st = finish_scatter(&p, vec, kTile)) != SWRT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (xf)
    return p.n == 1 ? dispatch<1, true>(p, vec, vmask, s)
                    : dispatch<kMaxTensors, true>(p, vec, vmask, s);
  return p.n == 1 ? dispatch<1, false>(p, vec, 0, s) : dispatch<kMaxTensors, false>(p, vec, 0, s);
}

}  // namespace

// ---------------------------------------------------------------------------
// plans (declared in swrt_host.hpp)
// ---------------------------------------------------------------------------
int plan_scatter(int n_tensors, void *const *presents, const void *const *pasts,
                 const void *const *updates, const int64_t *write_indices, const int64_t *shape,
                 int rank, int axis, int64_t seq_len, int mode, int elem_bits, uint32_t *d_flags,
                 const RowXf *xf, ScatterPlan *p, Range *ranges, int *nr) {
  p->empty = true;
  p->n = n_tensors;
  p->xf = xf ? *xf : RowXf{};
  if (n_tensors < 0 || n_tensors > kMaxTensors) return SWRT_E_INVALID_ARG;
  if (!shape || rank < 2 || rank > SWRT_MAX_RANK) return SWRT_E_INVALID_ARG;
  for (int d = 0; d < rank; ++d)
    if (shape[d] < 0) return SWRT_E_INVALID_ARG;
  if (axis < 0) axis += rank;
  if (axis < 1 || axis >= rank) return SWRT_E_INVALID_ARG;  // never the batch axis
  if (xf && axis != rank - 2) return SWRT_E_INVALID_ARG;     // a row is one head_dim
  if (mode != SWRT_MODE_LINEAR && mode != SWRT_MODE_CIRCULAR) return SWRT_E_INVALID_ARG;
  if (!valid_elem_bits(elem_bits)) return SWRT_E_INVALID_ARG;
  const int64_t M = shape[axis], S = seq_len, B = shape[0];
  if (S < 0 || S > M) return SWRT_E_INVALID_ARG;

  int64_t O = 1, I = 1, row_bits, n_rows, upd_rows;
  for (int d = 0; d < axis; ++d)
    if (!mul_ok(O, shape[d], &O)) return SWRT_E_UNSUPPORTED;
  for (int d = axis + 1; d < rank; ++d)
    if (!mul_ok(I, shape[d], &I)) return SWRT_E_UNSUPPORTED;
  if (!mul_ok(I, elem_bits, &row_bits)) return SWRT_E_UNSUPPORTED;
  if (row_bits % 8) return SWRT_E_UNSUPPORTED;  // 4-bit rows must end on a byte
  const int64_t row = row_bits / 8;
  int64_t cache_bytes, upd_bytes;
  if (!mul_ok(O, M, &n_rows) || !mul_ok(n_rows, row, &cache_bytes)) return SWRT_E_UNSUPPORTED;
  // update rows: the cache's elements, or the fused append's input elements
  const int64_t upd_row = xf ? I * xf->in_bytes : row;
  if (upd_row >= (int64_t(1) << 32)) return SWRT_E_UNSUPPORTED;
  if (!mul_ok(O, S, &upd_rows) || !mul_ok(upd_rows, upd_row, &upd_bytes)) return SWRT_E_UNSUPPORTED;
  if (n_tensors == 0 || cache_bytes == 0) return SWRT_OK;
  if (!presents || !pasts || (upd_bytes > 0 && !updates)) return SWRT_E_INVALID_ARG;

  // every tensor is in place, or every tensor is out of place
  const bool in_place = presents[0] == pasts[0];
  const uint64_t align = elem_align(elem_bits);
  const uint64_t upd_align = xf ? uint64_t(xf->in_bytes) : align;
  uint64_t acc = uint64_t(row);
  for (int t = 0; t < n_tensors; ++t) {
    const void *pr = presents[t], *pa = pasts[t], *up = upd_bytes > 0 ? updates[t] : nullptr;
    if (!pr || !pa || (upd_bytes > 0 && !up)) return SWRT_E_INVALID_ARG;
    if ((pr == pa) != in_place) return SWRT_E_INVALID_ARG;
    if (addr_of(pr) % align || addr_of(pa) % align || addr_of(up) % upd_align)
      return SWRT_E_INVALID_ARG;
    // fused-append updates are read element by element: not part of the word
    acc |= addr_of(pr) | addr_of(pa) | (xf ? 0 : addr_of(up));
    ranges[(*nr)++] = range(pr, uint64_t(cache_bytes), true);
    if (!in_place) ranges[(*nr)++] = range(pa, uint64_t(cache_bytes), false);
    ranges[(*nr)++] = range(up, uint64_t(upd_bytes), false);
    p->present[t] = static_cast<char *>(presents[t]);
    p->past[t] = static_cast<const char *>(pasts[t]);
    p->update[t] = static_cast<const char *>(up);
  }
  if (write_indices && addr_of(write_indices) % 8) return SWRT_E_INVALID_ARG;
  if (addr_of(d_flags) % 4) return SWRT_E_INVALID_ARG;
  ranges[(*nr)++] = range(write_indices, write_indices ? uint64_t(B) * 8 : 0, false);

  p->in_place = in_place;
  p->align = acc;
  p->row = row;
  p->rows = in_place ? upd_rows : n_rows;
  p->O = O;
  p->B = B;
  p->g.write_indices = write_indices;
  p->g.flags = d_flags;
  p->g.M = M;
  p->g.S = S;
  p->g.circular = mode == SWRT_MODE_CIRCULAR;
  p->g.in_row_bytes = uint32_t(upd_row);
  p->empty = in_place && upd_bytes == 0;
  return SWRT_OK;
}

int finish_scatter(ScatterPlan *p, int vec, uint32_t tile_words) {
  const int64_t words_per_row = p->row / vec;
  int64_t n_words;
  if (!mul_ok(p->rows, words_per_row, &n_words) || n_words >= (int64_t(1) << 31))
    return SWRT_E_UNSUPPORTED;
  const int64_t tiles = (n_words + tile_words - 1) / tile_words;
  if (tiles * p->n >= (int64_t(1) << 31)) return SWRT_E_UNSUPPORTED;
  p->tiles = uint32_t(tiles);
  p->g.n_words = uint32_t(n_words);
  p->g.words_per_row = uint32_t(words_per_row);
  p->g.by_row = FastDiv(uint32_t(words_per_row));
  p->g.by_seq = FastDiv(uint32_t(p->in_place ? p->g.S : p->g.M));
  p->g.by_batch = FastDiv(uint32_t(p->O / p->B));
  return SWRT_OK;
}

}  // namespace swrt

extern "C" int swrt_tensor_scatter(void *present, const void *past, const void *update,
                                   const int64_t *write_indices, const int64_t *shape, int rank,
                                   int axis, int64_t seq_len, int mode, int elem_bits,
                                   uint32_t *d_flags, void *stream) {
  return swrt::scatter(1, &present, &past, &update, write_indices, shape, rank, axis, seq_len,
                       mode, elem_bits, nullptr, nullptr, d_flags, stream);
}

extern "C" int swrt_tensor_scatter_batched(int n_tensors, void *const *presents,
                                           const void *const *pasts, const void *const *updates,
                                           const int64_t *write_indices, const int64_t *shape,
                                           int rank, int axis, int64_t seq_len, int mode,
                                           int elem_bits, uint32_t *d_flags, void *stream) {
  return swrt::scatter(n_tensors, presents, pasts, updates, write_indices, shape, rank, axis,
                       seq_len, mode, elem_bits, nullptr, nullptr, d_flags, stream);
}

extern "C" int swrt_tensor_scatter_xf(int n_tensors, void *const *presents,
                                      const void *const *pasts, const void *const *updates,
                                      const int *tensors, const int64_t *write_indices,
                                      const int64_t *shape, int rank, int64_t seq_len, int mode,
                                      const swrt_row_transform *xf, uint32_t *d_flags,
                                      void *stream) {
  if (!xf) return SWRT_E_INVALID_ARG;
  return swrt::scatter(n_tensors, presents, pasts, updates, write_indices, shape, rank, rank - 2,
                       seq_len, mode, 8, xf, tensors, d_flags, stream);
}
