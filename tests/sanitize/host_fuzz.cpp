// Randomized calls of every entry point of the library's C ABI, on a machine
// without a GPU, built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code (tests/test_sanitizers.py). Device pointers are made-up
// addresses that the host code never dereferences (they sit far apart, so
// distinct buffers do not overlap unless a case means them to); host arrays
// (shapes, strides, per-layer pointer arrays, layer descriptors, the
// transform) are heap blocks of exactly the documented length. Sizes are
// drawn from small values and from the extremes (0, -1, INT32_MAX,
// INT64_MAX ...), so the argument checks and the size arithmetic behind them
// run on overflowing inputs. A call that passes every check reaches its
// launch and fails there (no device): that is fine; an out-of-bounds host
// read or an undefined operation stops the run with a report.
#include <swrt.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {

uint64_t state = 0x9E3779B97F4A7C15ull;
uint64_t rnd() {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}
int64_t pick(int64_t lo, int64_t hi) { return lo + int64_t(rnd() % uint64_t(hi - lo + 1)); }

// a dimension or count: mostly small, sometimes an extreme
int dim() {
  static const int ext[] = {0, 1, 2, 3, 16, 64, 128, 4096, 65535, 1 << 20, INT32_MAX, -1, INT32_MIN};
  return rnd() % 4 ? int(pick(0, 70)) : ext[pick(0, 12)];
}
int64_t big() {
  static const int64_t ext[] = {0, 1, -1, 16, 4096, INT64_MAX, INT64_MIN, int64_t(1) << 40};
  return rnd() % 3 ? pick(0, 1 << 16) : ext[pick(0, 7)];
}

// made-up device addresses: buffer k at 2^44 + k * 2^36, 256-byte aligned,
// sometimes NULL, sometimes misaligned
int next_buf = 0;
void *dev() {
  const uint64_t r = rnd() % 16;
  if (r == 0) return nullptr;
  uint64_t a = (uint64_t(1) << 44) + uint64_t(next_buf++ % 4096) * (uint64_t(1) << 36);
  if (r == 1) a += pick(1, 15);
  return reinterpret_cast<void *>(a);
}
void *dev_same(void *p) { return rnd() % 8 ? dev() : p; }  // sometimes an overlap

struct Tally {
  long n[16] = {};
  void operator()(int st) { ++n[st >= 0 && st < 16 ? st : 15]; }
} tally;

template <class T>
T *host(size_t n) {  // exactly n elements (a 1-byte block for none)
  return static_cast<T *>(std::malloc(n ? n * sizeof(T) : 1));
}

std::vector<void *> dev_array(int n) {
  std::vector<void *> v;
  for (int i = 0; i < (n > 0 ? n : 0); ++i) v.push_back(dev());
  return v;
}
// a host array of n device pointers, exactly n long (NULL now and then for n > 0)
void **ptrs(int n, std::vector<void *> &keep) {
  keep = dev_array(n > 64 ? 0 : n);
  if (n > 0 && n <= 64 && rnd() % 20 == 0) return nullptr;
  void **p = host<void *>(keep.size());
  for (size_t i = 0; i < keep.size(); ++i) p[i] = keep[i];
  return p;
}
int small_n() { return rnd() % 6 ? int(pick(0, 4)) : dim(); }  // array lengths stay allocatable
int head_dim() { return rnd() % 2 ? int(16 << pick(0, 4)) : dim(); }  // the supported ones often

swrt_row_transform make_xf() {
  swrt_row_transform x;
  std::memset(&x, 0, sizeof(x));
  x.in_type = int(pick(0, 11));
  x.out_type = int(pick(0, 11));
  if (rnd() % 2) {
    x.cos_table = static_cast<const float *>(dev());
    x.sin_table = rnd() % 8 ? static_cast<const float *>(dev()) : nullptr;
    x.max_position = big();
    x.rotary_dim = rnd() % 2 ? 2 * pick(0, 40) : big();
    x.interleaved = int(pick(0, 2));
  }
  for (int t = 0; t < 2; ++t) {
    static const float sc[] = {1.0f, 0.5f, 0.0f, -1.0f, 1e30f, 3e38f};
    x.scale[t] = sc[pick(0, 5)];
    x.zero_point[t] = int32_t(pick(-300, 300));
    if (rnd() % 4 == 0) x.channel_scale[t] = static_cast<const float *>(dev());
    if (rnd() % 4 == 0) x.channel_zero_point[t] = static_cast<const int32_t *>(dev());
  }
  return x;
}

void call_scatter() {
  const int rank = int(pick(-1, 10));
  int64_t *shape = host<int64_t>(rank > 0 ? rank : 0);
  for (int d = 0; d < rank; ++d) shape[d] = rnd() % 5 ? pick(0, 40) : big();
  void *present = dev(), *past = rnd() % 2 ? present : dev();
  static const int bits[] = {4, 8, 16, 32, 64, 128, 0, 7, 256};
  tally(swrt_tensor_scatter(present, past, dev_same(present), static_cast<int64_t *>(dev()),
                            shape, rank, int(pick(-10, 10)), big(), int(pick(-1, 2)),
                            bits[pick(0, 8)], static_cast<uint32_t *>(dev()), nullptr));
  std::vector<void *> a, b, c;
  const int n = small_n();
  void **pr = ptrs(n, a), **pa = ptrs(n, b), **up = ptrs(n, c);
  if (pr && pa && rnd() % 2)
    for (size_t i = 0; i < a.size(); ++i) pa[i] = pr[i];
  tally(swrt_tensor_scatter_batched(n, pr, pa, up, static_cast<int64_t *>(dev()), shape, rank,
                                    int(pick(-3, 5)), big(), int(pick(0, 1)), bits[pick(0, 8)],
                                    static_cast<uint32_t *>(dev()), nullptr));
  swrt_row_transform x = make_xf();
  int *tensors = host<int>(a.size());
  for (size_t i = 0; i < a.size(); ++i) tensors[i] = int(pick(-1, 2));
  tally(swrt_tensor_scatter_xf(n, pr, pa, up, rnd() % 10 ? tensors : nullptr,
                               static_cast<int64_t *>(dev()), shape, rank, big(),
                               int(pick(0, 1)), rnd() % 10 ? &x : nullptr,
                               static_cast<uint32_t *>(dev()), nullptr));
  std::free(shape), std::free(pr), std::free(pa), std::free(up), std::free(tensors);
}

void call_lengths() {
  tally(swrt_kv_seq_lengths(static_cast<int32_t *>(dev()), dim(), dim(), dim(),
                            static_cast<int64_t *>(dev()), static_cast<int64_t *>(dev()),
                            static_cast<int32_t *>(dev()), static_cast<int32_t *>(dev()),
                            static_cast<int32_t *>(dev()), static_cast<int64_t *>(dev()),
                            static_cast<uint32_t *>(dev()), nullptr));
  tally(swrt_kv_seq_lengths_drift(static_cast<int32_t *>(dev()), dim(), dim(), dim(), dim(),
                                  static_cast<int64_t *>(dev()), static_cast<int64_t *>(dev()),
                                  static_cast<int32_t *>(dev()), static_cast<int32_t *>(dev()),
                                  static_cast<int32_t *>(dev()), static_cast<int64_t *>(dev()),
                                  static_cast<uint32_t *>(dev()), nullptr));
}

int64_t *strides3() {
  int64_t *s = host<int64_t>(3);
  for (int i = 0; i < 3; ++i) s[i] = rnd() % 4 ? pick(0, 5000) : big();
  return s;
}

void call_window() {
  static const int bits[] = {4, 8, 16, 32, 64, 128, 0, 12};
  int64_t *st = strides3();
  void *kc = dev(), *vc = dev_same(kc);
  tally(swrt_kv_window_append(kc, vc, dev(), dev(), rnd() % 10 ? st : nullptr, dev(), dev(),
                              static_cast<int32_t *>(dev()), static_cast<int32_t *>(dev()), dim(),
                              dim(), dim(), dim(), dim(), bits[pick(0, 7)], unsigned(pick(0, 4)),
                              static_cast<uint32_t *>(dev()), nullptr));
  tally(swrt_kv_window_append_noalloc(kc, vc, dev(), dev(), st, static_cast<int32_t *>(dev()),
                                      static_cast<int32_t *>(dev()), dim(), dim(), dim(), dim(),
                                      dim(), bits[pick(0, 7)], static_cast<uint32_t *>(dev()),
                                      nullptr));
  const int n = small_n();
  std::vector<void *> a, b, c, d, e, f;
  void **k = ptrs(n, a), **v = ptrs(n, b), **kn = ptrs(n, c), **vn = ptrs(n, d),
       **ks = ptrs(n, e), **vs = ptrs(n, f);
  tally(swrt_kv_window_append_layers(n, k, v, kn, vn, st, ks, vs, static_cast<int32_t *>(dev()),
                                     static_cast<int32_t *>(dev()), dim(), dim(), dim(), dim(),
                                     dim(), bits[pick(0, 7)], unsigned(pick(0, 4)),
                                     static_cast<uint32_t *>(dev()), nullptr));
  tally(swrt_kv_window_stage_step(n, k, v, kn, vn, st, ks, vs, static_cast<int32_t *>(dev()),
                                  dim(), dim(), static_cast<int64_t *>(dev()),
                                  static_cast<int64_t *>(dev()), static_cast<int32_t *>(dev()),
                                  static_cast<int32_t *>(dev()), static_cast<int32_t *>(dev()),
                                  dim(), dim(), dim(), dim(), bits[pick(0, 7)],
                                  static_cast<uint32_t *>(dev()), nullptr));
  swrt_row_transform x = make_xf();
  tally(swrt_kv_window_append_xf(n, k, v, kn, vn, st, ks, vs, static_cast<int32_t *>(dev()),
                                 static_cast<int32_t *>(dev()), static_cast<int64_t *>(dev()),
                                 dim(), dim(), dim(), dim(), dim(), unsigned(pick(0, 4)),
                                 rnd() % 10 ? &x : nullptr, static_cast<uint32_t *>(dev()),
                                 nullptr));
  tally(swrt_kv_window_stage_step_xf(n, k, v, kn, vn, st, ks, vs, static_cast<int32_t *>(dev()),
                                     dim(), dim(), static_cast<int64_t *>(dev()),
                                     static_cast<int64_t *>(dev()), static_cast<int32_t *>(dev()),
                                     static_cast<int32_t *>(dev()), static_cast<int32_t *>(dev()),
                                     dim(), dim(), dim(), dim(), &x,
                                     static_cast<uint32_t *>(dev()), nullptr));
  // the one-launch step: windowed layers and full caches
  const int nf = small_n();
  std::vector<void *> g, h, i2, j2;
  void **fk = ptrs(nf, g), **fv = ptrs(nf, h), **fkn = ptrs(nf, i2), **fvn = ptrs(nf, j2);
  tally(swrt_kv_decode_step(n, k, v, kn, vn, st, static_cast<int32_t *>(dev()), dim(), dim(),
                            static_cast<int64_t *>(dev()), static_cast<int64_t *>(dev()),
                            static_cast<int32_t *>(dev()), static_cast<int32_t *>(dev()),
                            static_cast<int32_t *>(dev()), nf, fk, fkn,
                            static_cast<int64_t *>(dev()), dim(), dim(), dim(), dim(),
                            bits[pick(0, 7)], static_cast<uint32_t *>(dev()), nullptr));
  tally(swrt_kv_decode_step_xf(n, k, v, kn, vn, st, static_cast<int32_t *>(dev()), dim(), dim(),
                               static_cast<int64_t *>(dev()), static_cast<int64_t *>(dev()),
                               static_cast<int32_t *>(dev()), static_cast<int32_t *>(dev()),
                               static_cast<int32_t *>(dev()), nf, fk, fv, fkn, fvn,
                               static_cast<int64_t *>(dev()), dim(), dim(), dim(), dim(), &x,
                               static_cast<uint32_t *>(dev()), nullptr));
  // windowed attention
  std::vector<void *> q, o;
  void **qs = ptrs(n, q), **os = ptrs(n, o);
  tally(swrt_window_attention(n, const_cast<const void *const *>(qs),
                              const_cast<const void *const *>(k),
                              const_cast<const void *const *>(v), os,
                              static_cast<int32_t *>(dev()), dim(), dim(), dim(), dim(), dim(),
                              dim(), rnd() % 8 ? 0.125f : -1.0f, int(pick(0, 11)),
                              int(pick(0, 11)), static_cast<uint32_t *>(dev()), nullptr));
  for (void **p : {k, v, kn, vn, ks, vs, fk, fv, fkn, fvn, qs, os}) std::free(p);
  std::free(st);
}

void call_paged() {
  const int n = small_n();
  const int nl = n > 0 && n <= 64 ? n : 0;
  swrt_paged_layer *L = host<swrt_paged_layer>(size_t(nl));
  for (int l = 0; l < nl; ++l) {
    L[l].q = dev();
    L[l].out = dev();
    L[l].arena = dev();
    L[l].arena_bytes = big();
    L[l].pages = static_cast<const swrt_page *>(dev());
    L[l].n_pages = big();
    L[l].page_ptr = static_cast<const int32_t *>(dev());
    L[l].page_ids = static_cast<const int32_t *>(dev());
    L[l].n_ids = big();
    L[l].page_count = rnd() % 2 ? static_cast<int32_t *>(dev()) : nullptr;
    L[l].page_stride = big();
    if (l > 0 && rnd() % 2) {  // a shared table
      L[l].pages = L[0].pages, L[l].page_ids = L[0].page_ids, L[l].page_ptr = L[0].page_ptr;
      L[l].page_count = L[0].page_count, L[l].n_pages = L[0].n_pages, L[l].n_ids = L[0].n_ids;
    }
  }
  static const uint32_t formats[] = {0u, (1u << 3) | (1u << 4), 0x3FEu, 1u, 1u << 12};
  tally(swrt_paged_attention(n, rnd() % 10 ? L : nullptr, big(), dim(), dim(), dim(), head_dim(),
                             0.125f, int(pick(0, 11)), int(pick(0, 11)), formats[pick(0, 4)],
                             static_cast<uint32_t *>(dev()), nullptr));
  tally(swrt_paged_quantize(dev(), big(), static_cast<const swrt_page *>(dev()), big(),
                            static_cast<const int32_t *>(dev()), big(),
                            static_cast<const int64_t *>(dev()), big(), big(),
                            static_cast<swrt_page *>(dev()), int(pick(0, 11)), 0.5f,
                            int32_t(pick(-10, 10)), int(pick(0, 11)), 0.25f,
                            int32_t(pick(-10, 10)), head_dim(), static_cast<uint32_t *>(dev()),
                            nullptr));
  std::vector<void *> a, b;
  void **kn = ptrs(nl, a), **vn = ptrs(nl, b);
  tally(swrt_paged_append(n, L, kn, vn, int(pick(0, 11)), dim(), dim(), head_dim(), big(), big(),
                          big(),
                          int(pick(0, 11)), 0.5f, int32_t(pick(-3, 3)), int(pick(0, 11)), 2.0f,
                          int32_t(pick(-3, 3)), static_cast<uint32_t *>(dev()), nullptr));
  tally(swrt_paged_append_open(n, L, kn, vn, int(pick(0, 11)), dim(), head_dim(),
                               static_cast<uint32_t *>(dev()), nullptr));
  std::free(L), std::free(kn), std::free(vn);
}

}  // namespace

int main(int argc, char **argv) {
  if (argc > 1 && std::strcmp(argv[1], "--overrun") == 0) {  // the sanitizer's own check
    volatile int64_t *p = host<int64_t>(3);
    p[3] = 1;
    std::free(const_cast<int64_t *>(p));
    return 0;
  }
  const long rounds = argc > 1 ? std::atol(argv[1]) : 2000;
  for (long r = 0; r < rounds; ++r) {
    call_scatter();
    call_lengths();
    call_window();
    call_paged();
  }
  for (int s = -8; s < 16; ++s) (void)swrt_status_string(s);
  std::printf("rounds %ld, abi %d: ok %ld, invalid %ld, unsupported %ld, launch %ld, other %ld\n",
              rounds, swrt_abi_version(), tally.n[SWRT_OK], tally.n[SWRT_E_INVALID_ARG],
              tally.n[SWRT_E_UNSUPPORTED], tally.n[SWRT_E_LAUNCH], tally.n[15]);
  return 0;
}
