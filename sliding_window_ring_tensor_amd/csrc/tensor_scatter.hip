// tensor_scatter.hip -- ONNX TensorScatter (operator page "TensorScatter",
// ai.onnx since version 24: description, pseudocode, Attributes) on gfx950.
//
// The cache is viewed as [O, M, I]: O = product of the dims before `axis`,
// M = shape[axis] (max_sequence_length), I = product of the dims after it.
// The update is [O, S, I]. Prefix o belongs to batch entry b = o / (O / B).
// Row (o, s) of the update goes to cache row j = w_b + s (linear) or
// (w_b + s) mod M (circular, floor modulo; the modulo applies to the sequence
// index only). A linear entry with w_b < 0 or w_b > M - S is flagged and its
// rows are left as in past.
//
// In place (present == past) only the O*S target rows move: one thread per
// raw-bit word of the update, consecutive threads on consecutive words, so the
// update is read and the target rows are written fully coalesced. Out of place
// every present row is produced in one pass from either past or the update.
#include "swrt_device.hpp"

namespace swrt {
namespace {

constexpr int kUnroll = 4;  // words per thread per tile

template <int NT>
struct ScatterArgs {
  char *present[NT];
  const char *past[NT];
  const char *update[NT];
  uint32_t tiles;                // tiles per tensor
  const int64_t *write_indices;  // [B] or null
  uint32_t *flags;
  int64_t M, S;
  uint32_t n_words;       // words to produce (update words in place, present words otherwise)
  uint32_t words_per_row;  // row bytes / VEC
  FastDiv by_row;          // words -> row
  FastDiv by_seq;          // row -> (o, s) in place; row -> (o, j) out of place
  FastDiv by_batch;        // o -> b
  int circular;
};

// floor modulo of a 64-bit index into [0, M); the division is skipped for the
// usual case of an index already in range.
__device__ __forceinline__ int64_t wrap(int64_t w, int64_t M) {
  if (w >= 0 && w < M) return w;
  int64_t r = w % M;
  return r < 0 ? r + M : r;
}

constexpr uint32_t kTile = kBlock * kUnroll;

// The write index of every batch entry this workgroup's tile touches, staged
// once in LDS (the tile's words span at most kTile + 1 entries). Circular
// entries hold w mod M; linear entries hold w, or -1 when the entry is out of
// range (then flagged). Lane lookups are LDS reads, so the only global loads
// of a lane are its payload words.
struct TileBatches {
  uint32_t first;
  int64_t w[kTile + 1];
};

template <int NT>
__device__ __forceinline__ int64_t reduce_write_index(const ScatterArgs<NT> &a, int64_t w) {
  if (a.circular) return wrap(w, a.M);
  if (w < 0 || w > a.M - a.S) {  // no partial update of this batch entry
    if (a.flags) atomicOr(a.flags, SWRT_FLAG_LINEAR_OOB);
    return -1;
  }
  return w;
}

// Staging runs in two halves around the payload loads: the first half issues
// the index loads (thread k fetches entry first + k), the second half waits
// for them, fills LDS and meets at a barrier. Vector memory counters retire
// in order, so index loads issued before the payload loads can be waited for
// without waiting for the payload.
struct WPrefetch {
  uint32_t first, count;
  int64_t w;
};

template <int NT>
__device__ __forceinline__ WPrefetch prefetch_write_indices(const ScatterArgs<NT> &a, uint32_t tile) {
  const uint32_t last = min(tile + kTile, a.n_words) - 1;
  WPrefetch p;
  p.first = a.by_batch.div(a.by_seq.div(a.by_row.div(tile)));
  p.count = a.by_batch.div(a.by_seq.div(a.by_row.div(last))) - p.first + 1;
  const uint32_t k = min(threadIdx.x, p.count - 1);
  p.w = a.write_indices ? a.write_indices[p.first + k] : 0;
  return p;
}

template <int NT>
__device__ __forceinline__ void finish_write_indices(const ScatterArgs<NT> &a, const WPrefetch &p,
                                                     TileBatches &tb) {
  if (threadIdx.x == 0) tb.first = p.first;
  if (threadIdx.x < p.count) tb.w[threadIdx.x] = reduce_write_index(a, p.w);
  for (uint32_t k = threadIdx.x + kBlock; k < p.count; k += kBlock)  // many tiny rows
    tb.w[k] = reduce_write_index(a, a.write_indices ? a.write_indices[p.first + k] : 0);
  __syncthreads();
}

// Lanes past the last word clamp to it (they repeat that lane's load and
// store), so the loops carry no per-lane branch except the linear
// out-of-range skip, which only guards stores.
template <int VEC, int NT>
__global__ __launch_bounds__(kBlock) void scatter_in_place(ScatterArgs<NT> a) {
  using W = typename Word<VEC>::T;
  __shared__ TileBatches tb;
  const uint32_t t = blockIdx.x / a.tiles;  // which tensor of a batched call
  const uint32_t tile = (blockIdx.x - t * a.tiles) * kTile;
  const WPrefetch wp = prefetch_write_indices(a, tile);
  const W *update = reinterpret_cast<const W *>(a.update[t]);
  W *present = reinterpret_cast<W *>(a.present[t]);
  W v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) v[u] = ld(update + min(tile + u * kBlock + threadIdx.x, a.n_words - 1));
  finish_write_indices(a, wp, tb);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t i = min(tile + u * kBlock + threadIdx.x, a.n_words - 1);
    const uint32_t row = a.by_row.div(i);
    const uint32_t col = i - row * a.words_per_row;
    const uint32_t o = a.by_seq.div(row);
    const uint32_t s = row - o * uint32_t(a.S);
    const int64_t w = tb.w[a.by_batch.div(o) - tb.first];
    int64_t j = w + s;
    if (a.circular && j >= a.M) j -= a.M;
    if (w >= 0) st(present + (int64_t(o) * a.M + j) * a.words_per_row + col, v[u]);
  }
}

template <int VEC, int NT>
__global__ __launch_bounds__(kBlock) void scatter_out_of_place(ScatterArgs<NT> a) {
  using W = typename Word<VEC>::T;
  __shared__ TileBatches tb;
  const uint32_t t = blockIdx.x / a.tiles;
  const uint32_t tile = (blockIdx.x - t * a.tiles) * kTile;
  finish_write_indices(a, prefetch_write_indices(a, tile), tb);
  const W *update = reinterpret_cast<const W *>(a.update[t]);
  const W *past = reinterpret_cast<const W *>(a.past[t]);
  W *present = reinterpret_cast<W *>(a.present[t]);
  W v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t i = min(tile + u * kBlock + threadIdx.x, a.n_words - 1);
    const uint32_t row = a.by_row.div(i);
    const uint32_t col = i - row * a.words_per_row;
    const uint32_t o = a.by_seq.div(row);
    const int64_t j = row - o * uint32_t(a.M);
    const int64_t w = tb.w[a.by_batch.div(o) - tb.first];
    int64_t s = -1;  // the update row landing on (o, j), if any
    if (w >= 0) {
      s = j - w;
      if (a.circular && s < 0) s += a.M;
      if (s >= a.S) s = -1;
    }
    v[u] = ld(s >= 0 ? update + (int64_t(o) * a.S + s) * a.words_per_row + col : past + i);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) st(present + min(tile + u * kBlock + threadIdx.x, a.n_words - 1), v[u]);
}

template <int VEC, int NT>
int launch(ScatterArgs<NT> a, int n_tensors, bool in_place, hipStream_t stream) {
  a.tiles = (a.n_words + kTile - 1) / kTile;
  const dim3 grid(a.tiles * uint32_t(n_tensors));
  if (in_place)
    hipLaunchKernelGGL((scatter_in_place<VEC, NT>), grid, dim3(kBlock), 0, stream, a);
  else
    hipLaunchKernelGGL((scatter_out_of_place<VEC, NT>), grid, dim3(kBlock), 0, stream, a);
  return launch_status();
}

template <int NT>
int dispatch(const ScatterArgs<NT> &a, int vec, int n_tensors, bool in_place, hipStream_t s) {
  switch (vec) {
    case 16: return launch<16>(a, n_tensors, in_place, s);
    case 8: return launch<8>(a, n_tensors, in_place, s);
    case 4: return launch<4>(a, n_tensors, in_place, s);
    case 2: return launch<2>(a, n_tensors, in_place, s);
    default: return launch<1>(a, n_tensors, in_place, s);
  }
}

constexpr int kMaxTensors = SWRT_MAX_BATCHED;

// Validation and launch shared by the single and the batched entry point.
int scatter(int n_tensors, void *const *presents, const void *const *pasts,
            const void *const *updates, const int64_t *write_indices, const int64_t *shape,
            int rank, int axis, int64_t seq_len, int mode, int elem_bits, uint32_t *d_flags,
            void *stream) {
  if (n_tensors < 0 || n_tensors > kMaxTensors) return SWRT_E_INVALID_ARG;
  if (!shape || rank < 2 || rank > SWRT_MAX_RANK) return SWRT_E_INVALID_ARG;
  for (int d = 0; d < rank; ++d)
    if (shape[d] < 0) return SWRT_E_INVALID_ARG;
  if (axis < 0) axis += rank;
  if (axis < 1 || axis >= rank) return SWRT_E_INVALID_ARG;  // never the batch axis
  if (mode != SWRT_MODE_LINEAR && mode != SWRT_MODE_CIRCULAR) return SWRT_E_INVALID_ARG;
  if (!valid_elem_bits(elem_bits)) return SWRT_E_INVALID_ARG;
  const int64_t M = shape[axis], S = seq_len, B = shape[0];
  if (S < 0 || S > M) return SWRT_E_INVALID_ARG;

  int64_t O = 1, I = 1, row_bits, n_rows, upd_rows, row_bytes;
  for (int d = 0; d < axis; ++d)
    if (!mul_ok(O, shape[d], &O)) return SWRT_E_UNSUPPORTED;
  for (int d = axis + 1; d < rank; ++d)
    if (!mul_ok(I, shape[d], &I)) return SWRT_E_UNSUPPORTED;
  if (!mul_ok(I, elem_bits, &row_bits)) return SWRT_E_UNSUPPORTED;
  if (row_bits % 8) return SWRT_E_UNSUPPORTED;  // 4-bit rows must end on a byte
  row_bytes = row_bits / 8;
  int64_t cache_bytes, upd_bytes;
  if (!mul_ok(O, M, &n_rows) || !mul_ok(n_rows, row_bytes, &cache_bytes)) return SWRT_E_UNSUPPORTED;
  if (!mul_ok(O, S, &upd_rows) || !mul_ok(upd_rows, row_bytes, &upd_bytes)) return SWRT_E_UNSUPPORTED;
  if (n_tensors == 0 || cache_bytes == 0) return SWRT_OK;
  if (!presents || !pasts || (upd_bytes > 0 && !updates)) return SWRT_E_INVALID_ARG;

  // every tensor is in place, or every tensor is out of place
  const bool in_place = presents[0] == pasts[0];
  const auto addr = [](const void *p) { return uint64_t(reinterpret_cast<uintptr_t>(p)); };
  const uint64_t align = elem_bits >= 16 ? uint64_t(elem_bits / 8 > 8 ? 8 : elem_bits / 8) : 1;
  uint64_t align_acc = uint64_t(row_bytes);
  Range ranges[3 * kMaxTensors + 2];
  int nr = 0;
  ScatterArgs<kMaxTensors> a = {};
  for (int t = 0; t < n_tensors; ++t) {
    const void *pr = presents[t], *pa = pasts[t], *up = upd_bytes > 0 ? updates[t] : nullptr;
    if (!pr || !pa || (upd_bytes > 0 && !up)) return SWRT_E_INVALID_ARG;
    if ((pr == pa) != in_place) return SWRT_E_INVALID_ARG;
    if (addr(pr) % align || addr(pa) % align || addr(up) % align) return SWRT_E_INVALID_ARG;
    align_acc |= addr(pr) | addr(pa) | addr(up);
    ranges[nr++] = range(pr, uint64_t(cache_bytes), true);
    if (!in_place) ranges[nr++] = range(pa, uint64_t(cache_bytes), false);
    ranges[nr++] = range(up, uint64_t(upd_bytes), false);
    a.present[t] = static_cast<char *>(presents[t]);
    a.past[t] = static_cast<const char *>(pasts[t]);
    a.update[t] = static_cast<const char *>(up);
  }
  if (write_indices && addr(write_indices) % 8) return SWRT_E_INVALID_ARG;
  if (d_flags && addr(d_flags) % 4) return SWRT_E_INVALID_ARG;
  ranges[nr++] = range(write_indices, write_indices ? uint64_t(B) * 8 : 0, false);
  ranges[nr++] = range(d_flags, 4, true);
  if (written_overlap(ranges, nr)) return SWRT_E_INVALID_ARG;
  if (in_place && upd_bytes == 0) return SWRT_OK;

  const int vec = align_acc % 16 == 0 ? 16 : align_acc % 8 == 0 ? 8 : align_acc % 4 == 0 ? 4
                : align_acc % 2 == 0 ? 2 : 1;
  const int64_t words_per_row = row_bytes / vec;
  const int64_t n_words = (in_place ? upd_rows : n_rows) * words_per_row;
  const int64_t tiles = (n_words + kTile - 1) / kTile;
  if (n_words >= (int64_t(1) << 31) || tiles * n_tensors >= (int64_t(1) << 31))
    return SWRT_E_UNSUPPORTED;

  a.write_indices = write_indices;
  a.flags = d_flags;
  a.M = M;
  a.S = S;
  a.n_words = uint32_t(n_words);
  a.words_per_row = uint32_t(words_per_row);
  a.by_row = FastDiv(uint32_t(words_per_row));
  a.by_seq = FastDiv(uint32_t(in_place ? S : M));
  a.by_batch = FastDiv(uint32_t(O / B));
  a.circular = mode == SWRT_MODE_CIRCULAR;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n_tensors == 1) {
    ScatterArgs<1> one;
    one.present[0] = a.present[0];
    one.past[0] = a.past[0];
    one.update[0] = a.update[0];
    one.tiles = 1;
    one.write_indices = a.write_indices;
    one.flags = a.flags;
    one.M = a.M;
    one.S = a.S;
    one.n_words = a.n_words;
    one.words_per_row = a.words_per_row;
    one.by_row = a.by_row;
    one.by_seq = a.by_seq;
    one.by_batch = a.by_batch;
    one.circular = a.circular;
    return dispatch(one, vec, 1, in_place, s);
  }
  return dispatch(a, vec, n_tensors, in_place, s);
}

}  // namespace
}  // namespace swrt

extern "C" int swrt_tensor_scatter(void *present, const void *past, const void *update,
                                   const int64_t *write_indices, const int64_t *shape, int rank,
                                   int axis, int64_t seq_len, int mode, int elem_bits,
                                   uint32_t *d_flags, void *stream) {
  return swrt::scatter(1, &present, &past, &update, write_indices, shape, rank, axis, seq_len,
                       mode, elem_bits, d_flags, stream);
}

extern "C" int swrt_tensor_scatter_batched(int n_tensors, void *const *presents,
                                           const void *const *pasts, const void *const *updates,
                                           const int64_t *write_indices, const int64_t *shape,
                                           int rank, int axis, int64_t seq_len, int mode,
                                           int elem_bits, uint32_t *d_flags, void *stream) {
  return swrt::scatter(n_tensors, presents, pasts, updates, write_indices, shape, rank, axis,
                       seq_len, mode, elem_bits, d_flags, stream);
}
