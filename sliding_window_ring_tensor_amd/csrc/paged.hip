// paged.hip -- paged caches with per-page formats on gfx950 (onnx-light how-to
// "Persistent input/output feedback", section "Optional heterogeneous paged
// KV": pages with start, length and capacity, contiguous from zero; dense
// FLOAT / FLOAT16 / BFLOAT16 or affine INT8 / UINT8 / INT4 / UINT4 / INT2 /
// UINT2 payloads per page, independently for K and V; QuantizePagedCache on
// selected blocks; attention over the visible tokens only, with online
// softmax and a left window bounding the preceding tokens).
//
// Four kernel families:
//   paged_attention_kernel  one wave per (layer, batch entry, KV head) stream
//                           and chunk of 16 query heads, each layer's
//                           workgroups aligned to the eight XCDs:
//                           finds the pages its window reaches, checks each,
//                           stages each 16-row tile of a page into LDS as it
//                           lies in the page, decodes it in the page's formats
//                           and runs both contractions on the matrix cores
//                           with exact operands (bf16 values and affine codes
//                           as the exact integers c - zp on the bf16
//                           instructions, fp32 weights as three exact bf16
//                           parts; fp32 and f16 pages on the fp32 ones), the
//                           scales applied to the score and the weight. Built
//                           per declared format set: bf16 and int8 pages
//                           only (a tile loop of its own, six waves per SIMD
//                           at head_dim 64), every staged format but f16, or
//                           all formats.
//   paged_validate / paged_convert / paged_publish
//                           the conversion of selected pages: every check on
//                           the device first, then the payloads, then the
//                           descriptors, each later kernel stopping when the
//                           first raised the flag.
//   paged_append_sealed     one wave per (block table, stream): the stream's
//                           new tokens as one new block (the pages' sealed
//                           rule), every layer's payload encoded, then the
//                           block's descriptor and the table slot.
//   paged_append_rows / paged_append_commit
//                           the open-page extension: one wave per (layer,
//                           stream) writes the new token into the last page,
//                           then, once per distinct table, its length + 1.
#include "swrt_host.hpp"
#include "att_device.hpp"

namespace swrt {
namespace {

constexpr int kPgBlock = 128;  // 2 waves, one stream each (4 measured 0.2 us slower)
constexpr int kPgWaves = kPgBlock / 64;

static_assert(sizeof(swrt_paged_layer) == 88, "swrt_paged_layer layout");

struct PgLayer {
  const char *q;
  char *out;
  const char *arena;
  int64_t arena_bytes;
  const swrt_page *pages;
  int64_t n_pages;
  const int32_t *page_ptr;
  const int32_t *page_ids;
  int64_t n_ids;
  int32_t *page_count;  // slotted rows (null: compressed rows through page_ptr)
  int64_t page_stride;
};

// ---------------------------------------------------------------------------
// formats
// ---------------------------------------------------------------------------
// Format properties as table lookups (a chain of comparisons on a run-time
// format would compile to a chain of branches). Nibble f of kPgLogBits is
// log2 of format f's element bits (0: not a format): F32 5, F16 and BF16 4,
// INT8 and UINT8 3, INT4 and UINT4 2, INT2 and UINT2 1.
constexpr uint64_t kPgLogBits = 0x1122334450ull;
__host__ __device__ constexpr int pg_bits(int f) {
  return f >= 0 && f <= SWRT_XF_UINT2 && ((kPgLogBits >> (4 * f)) & 15) != 0
             ? 1 << ((kPgLogBits >> (4 * f)) & 15)
             : 0;
}
__host__ __device__ constexpr bool pg_affine(int f) { return f >= SWRT_XF_INT8 && f <= SWRT_XF_UINT2; }
__host__ __device__ constexpr bool pg_signed(int f) {  // INT8, INT4, INT2: bits 4, 6, 8
  return f >= 0 && f <= SWRT_XF_UINT2 && ((0x150u >> f) & 1u) != 0;
}
static_assert(pg_bits(SWRT_XF_F32) == 32 && pg_bits(SWRT_XF_F16) == 16 && pg_bits(SWRT_XF_BF16) == 16 &&
                  pg_bits(SWRT_XF_INT8) == 8 && pg_bits(SWRT_XF_UINT8) == 8 && pg_bits(SWRT_XF_INT4) == 4 &&
                  pg_bits(SWRT_XF_UINT4) == 4 && pg_bits(SWRT_XF_INT2) == 2 && pg_bits(SWRT_XF_UINT2) == 2 &&
                  pg_bits(0) == 0 && pg_bits(10) == 0,
              "format bits");
static_assert(pg_signed(SWRT_XF_INT8) && pg_signed(SWRT_XF_INT4) && pg_signed(SWRT_XF_INT2) &&
                  !pg_signed(SWRT_XF_UINT8) && !pg_signed(SWRT_XF_UINT4) && !pg_signed(SWRT_XF_UINT2) &&
                  !pg_signed(SWRT_XF_BF16),
              "signed formats");
__host__ __device__ constexpr int32_t pg_lo(int f) { return pg_signed(f) ? -(1 << (pg_bits(f) - 1)) : 0; }
__host__ __device__ constexpr int32_t pg_hi(int f) {
  return pg_signed(f) ? (1 << (pg_bits(f) - 1)) - 1 : (1 << pg_bits(f)) - 1;
}

// a format with its parameters (an affine one: positive finite scale, zero
// point inside the code range)
__host__ __device__ inline bool pg_format_ok(int f, float scale, int32_t zp) {
  if (pg_bits(f) == 0) return false;
  if (!pg_affine(f)) return true;
  return scale > 0.0f && scale <= 3.4028235e38f && zp >= pg_lo(f) && zp <= pg_hi(f);
}

__host__ __device__ inline int64_t pg_row_bytes(int f, int D) { return int64_t(D) * pg_bits(f) / 8; }

// [off, off + bytes) inside [0, arena), off 16-byte aligned
__device__ __forceinline__ bool pg_inside(int64_t off, int64_t bytes, int64_t arena) {
  return off >= 0 && (off & 15) == 0 && off <= arena && bytes <= arena - off;
}

__device__ __forceinline__ bool pg_page_ok(const swrt_page &p, int D, int64_t arena) {
  if (p.start < 0 || p.capacity < 1 || p.length < 1 || p.length > p.capacity) return false;
  if (!pg_format_ok(p.k_format, p.k_scale, p.k_zero_point) ||
      !pg_format_ok(p.v_format, p.v_scale, p.v_zero_point))
    return false;
  if (p.start > INT64_MAX - p.length) return false;
  return pg_inside(p.k_offset, p.capacity * pg_row_bytes(p.k_format, D), arena) &&
         pg_inside(p.v_offset, p.capacity * pg_row_bytes(p.v_format, D), arena);
}

// a descriptor read whole with uniform (scalar) loads
__device__ __forceinline__ swrt_page pg_read(const swrt_page *pages, int32_t id) {
  return pages[__builtin_amdgcn_readfirstlane(id)];
}

// Stream s's slots of the block table, [p0, p1) of page_ids: compressed rows
// page_ptr[s] .. page_ptr[s + 1], or slotted rows s * page_stride +
// [0, page_count[s]). False when the range does not lie inside page_ids.
// UNIFORM: s is the same in every lane, the loads are scalar.
template <bool UNIFORM = true>
__device__ __forceinline__ bool pg_stream_range(const PgLayer &P, int64_t s, int64_t &p0, int64_t &p1) {
  auto u = [](int32_t v) { return UNIFORM ? __builtin_amdgcn_readfirstlane(v) : v; };
  if (P.page_count) {
    const int64_t n = u(P.page_count[s]);
    p0 = s * P.page_stride;
    p1 = p0 + n;
    return n >= 0 && n <= P.page_stride && P.page_stride <= P.n_ids - p0;
  }
  p0 = u(P.page_ptr[s]);
  p1 = u(P.page_ptr[s + 1]);
  return p0 >= 0 && p0 <= p1 && p1 <= P.n_ids;
}

// Payload addresses computed as integers are turned back into pointers to
// global memory, never generic ones: a generic load also counts on the
// counter that cross-lane shuffles and scalar loads wait on, so every such
// wait would stall until all payload loads in flight had landed.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T *pg_g(uintptr_t a) {
  return (const __attribute__((address_space(1))) T *)a;
}
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T *pg_g(const T *p) {
  return (const __attribute__((address_space(1))) T *)p;
}
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T *pg_gw(T *p) {
  return (__attribute__((address_space(1))) T *)p;
}

// NB bytes (1, 2, 4, 8 or a multiple of 16) of a payload as 32-bit words
template <int NB>
__device__ __forceinline__ void pg_load_raw(const char *p, uint32_t (&w)[(NB + 3) / 4]) {
  if constexpr (NB == 1) {
    w[0] = __builtin_nontemporal_load(pg_g(reinterpret_cast<const uint8_t *>(p)));
  } else if constexpr (NB == 2) {
    w[0] = __builtin_nontemporal_load(pg_g(reinterpret_cast<const uint16_t *>(p)));
  } else if constexpr (NB == 4) {
    w[0] = __builtin_nontemporal_load(pg_g(reinterpret_cast<const uint32_t *>(p)));
  } else if constexpr (NB == 8) {
    const u32x2 x = __builtin_nontemporal_load(pg_g(reinterpret_cast<const u32x2 *>(p)));
    w[0] = x.x;
    w[1] = x.y;
  } else {
    static_assert(NB % 16 == 0, "payload chunk");
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const u32x4 x = __builtin_nontemporal_load(pg_g(reinterpret_cast<const u32x4 *>(p) + i));
      w[4 * i] = x.x;
      w[4 * i + 1] = x.y;
      w[4 * i + 2] = x.z;
      w[4 * i + 3] = x.w;
    }
  }
}

// element e of packed words as binary32: a dense value, or the exact integer
// c - zp of an affine code (its scale applied by the caller). ZP false: the
// page's zero point is 0 (a uniform test per page), and the code is the value.
template <int FMT, bool ZP = true>
__device__ __forceinline__ float pg_elem(const uint32_t *w, int e, int32_t zp) {
  if constexpr (FMT == SWRT_XF_F32) {
    return __uint_as_float(w[e]);
  } else if constexpr (FMT == SWRT_XF_BF16) {
    return __uint_as_float(e & 1 ? w[e / 2] & 0xFFFF0000u : w[e / 2] << 16);
  } else if constexpr (FMT == SWRT_XF_F16) {
    return float(__builtin_bit_cast(_Float16, uint16_t(w[e / 2] >> (16 * (e & 1)))));
  } else if constexpr (FMT == SWRT_XF_UINT8) {
    const float c = float((w[e / 4] >> (8 * (e % 4))) & 0xFFu);  // a byte conversion, exact
    return ZP ? c - float(zp) : c;
  } else if constexpr (FMT == SWRT_XF_INT8) {
    const float c = float(int(int8_t(w[e / 4] >> (8 * (e % 4)))));  // a sign-extending byte conversion
    return ZP ? c - float(zp) : c;
  } else {
    constexpr int B = pg_bits(FMT);
    const uint32_t raw = (w[e * B / 32] >> (e * B % 32)) & ((1u << B) - 1u);
    int32_t c = int32_t(raw);
    if constexpr (pg_signed(FMT)) c = int32_t(raw << (32 - B)) >> (32 - B);
    return float(c - zp);
  }
}


// N elements starting at element `first` of a row, decoded (see pg_elem)
template <int N, int FMT>
__device__ __forceinline__ void pg_load_decode_t(const char *row, uint32_t first, int32_t zp,
                                                 float (&out)[N]) {
  constexpr int B = pg_bits(FMT);
  constexpr int NB = N * B / 8 > 0 ? N * B / 8 : 1;
  uint32_t w[(NB + 3) / 4];
  const uint32_t bit = first * B;
  pg_load_raw<NB>(row + bit / 8, w);
  if constexpr (N * B < 8) w[0] >>= bit % 8;  // a sub-byte chunk: its place in the byte
#pragma unroll
  for (int e = 0; e < N; ++e) out[e] = pg_elem<FMT>(w, e, zp);
}

template <int N>
__device__ __forceinline__ void pg_load_decode(int fmt, const char *row, uint32_t first, int32_t zp,
                                               float (&out)[N]) {
  switch (fmt) {  // uniform in the wave
    case SWRT_XF_F32: pg_load_decode_t<N, SWRT_XF_F32>(row, first, zp, out); break;
    case SWRT_XF_F16: pg_load_decode_t<N, SWRT_XF_F16>(row, first, zp, out); break;
    case SWRT_XF_BF16: pg_load_decode_t<N, SWRT_XF_BF16>(row, first, zp, out); break;
    case SWRT_XF_INT8: pg_load_decode_t<N, SWRT_XF_INT8>(row, first, zp, out); break;
    case SWRT_XF_UINT8: pg_load_decode_t<N, SWRT_XF_UINT8>(row, first, zp, out); break;
    case SWRT_XF_INT4: pg_load_decode_t<N, SWRT_XF_INT4>(row, first, zp, out); break;
    case SWRT_XF_UINT4: pg_load_decode_t<N, SWRT_XF_UINT4>(row, first, zp, out); break;
    case SWRT_XF_INT2: pg_load_decode_t<N, SWRT_XF_INT2>(row, first, zp, out); break;
    default: pg_load_decode_t<N, SWRT_XF_UINT2>(row, first, zp, out); break;
  }
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct PgAttArgs {
  PgLayer L[kMaxLayers];
  uint32_t *flags;
  float scale_log2;  // scale * log2(e)
  int64_t left_window;
  int32_t B, Hq, Hkv, q_type, out_type;
  int32_t items;     // per layer: (stream, chunk) pairs
  int32_t wg_layer;  // workgroups per layer, a multiple of the 8 XCDs
  int32_t chunks;    // groups of up to 16 query heads per KV head
  uint32_t formats;  // bit f set: pages of format f are allowed
};

// A tile is up to 16 consecutive rows of one page, staged in LDS as they lie
// in the page: 16 K rows, then 16 V rows, of up to 16 bits per element (an
// fp32 page is read from memory by its own tile code). Each lane then reads
// exactly its chunks: the K chunk of row pk, elements [q D/4, (q + 1) D/4),
// and the V chunks of rows 4 c + q, elements [MT j, MT (j + 1)). Up to
// head_dim 128 the next tile's rows are staged while this one is computed:
// the general tile loop keeps two buffers of K and V, the bf16 + int8 one a
// K buffer (refilled as soon as the tile's K chunks are read out) and two of
// V.
template <int D>
struct PgStage {
  static constexpr int BYTES = 16 * D * 2;       // one tile's K (or V) rows
  static constexpr int NBUF = D <= 128 ? 2 : 1;  // buffers per wave
  static constexpr int LG_D = D == 32 ? 5 : D == 64 ? 6 : D == 128 ? 7 : 8;
  static_assert((1 << LG_D) == D, "head_dim");
};

// One lane's query operand: head slot j's D/4 dimensions of lane group q, as
// bf16 pairs for a bf16 query (the values are exactly bf16), else in binary32.
template <int D, bool QBF>
struct PgQuery;
template <int D>
struct PgQuery<D, true> {
  uint32_t b[D / 8];
  __device__ __forceinline__ void set(const float (&v)[D / 4]) {
#pragma unroll
    for (int i = 0; i < D / 8; ++i)
      b[i] = (__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u);
  }
  __device__ __forceinline__ float f(int e) const {
    return __uint_as_float(e & 1 ? b[e / 2] & 0xFFFF0000u : b[e / 2] << 16);
  }
};
template <int D>
struct PgQuery<D, false> {
  float v[D / 4];
  __device__ __forceinline__ void set(const float (&x)[D / 4]) {
#pragma unroll
    for (int i = 0; i < D / 4; ++i) v[i] = x[i];
  }
  __device__ __forceinline__ float f(int e) const { return v[e]; }
};

// Payload staged straight into LDS, without passing through registers: lane
// l's 16 (or 4) bytes land at dst + 16 l (dst + 4 l); the wave's
// vector-memory counter covers the copy.
typedef const __attribute__((address_space(1))) char *pg_gchar;
__device__ __forceinline__ void pg_stage16(pg_gchar src, char *dst) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)src,
                                   (__attribute__((address_space(3))) void *)dst, 16, 0,
                                   2 /* non-temporal */);
}
__device__ __forceinline__ void pg_stage4(pg_gchar src, char *dst) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)src,
                                   (__attribute__((address_space(3))) void *)dst, 4, 0,
                                   2 /* non-temporal */);
}

// Rows [i, i + 16) of a page's payload (rows of 2^lg_rb bytes, 8 to 512) to
// LDS at dst, as they lie in the page. Byte o of the tile comes from row
// i + o / row bytes; rows past the page's last (lim rows after row i) repeat
// that row, so every load stays inside the page (scores of such rows are
// masked). The page's row i is the uniform base; a lane adds a 32-bit offset.
template <int NMAX>
__device__ __forceinline__ void pg_stage_rows(const char *page, int32_t i, int32_t lim, int lg_rb,
                                              char *dst, uint32_t lane) {
  const pg_gchar base = pg_gchar(page) + (int64_t(i) << lg_rb);
  if (lg_rb >= 4) {
    const int n = lg_rb >= 6 ? 1 << (lg_rb - 6) : 1;  // 16 rows in 1 KiB instructions, at most NMAX
    const uint32_t in_row = (1u << lg_rb) - 1;
#pragma unroll
    for (int k = 0; k < NMAX; ++k) {
      if (k > 0 && k >= n) break;  // uniform
      const uint32_t o = uint32_t(k) * 1024 + lane * 16;
      const uint32_t rr = uint32_t(min(int32_t(o >> lg_rb), lim));
      pg_stage16(base + ((rr << lg_rb) | (o & in_row)), dst + k * 1024);
    }
  } else {  // 8-byte rows: 128 bytes, four per lane (lanes past 31 repeat the last row)
    const uint32_t o = min(lane, 31u) * 4;
    const uint32_t rr = uint32_t(min(int32_t(o >> 3), lim));
    pg_stage4(base + ((rr << 3) | (o & 7)), dst);
  }
}

// A tile of a bf16 (rows of 2D bytes) or int8 (D bytes) payload to LDS at
// dst: 16 rows from src, or the `rows` left (fewer than 16: the last one
// repeats). A whole tile of 1 KiB pieces is copied as it lies, with no
// per-lane clamp.
template <int D>
__device__ __forceinline__ void pg_stage_lean(int64_t src, int32_t rows, bool is8, char *dst,
                                              uint32_t lane) {
  constexpr int N8 = 16 * D / 1024, N16 = 32 * D / 1024;  // 1 KiB pieces of a whole tile
  if (rows >= 16 && (N8 > 0 || !is8)) {
    const pg_gchar base = pg_gchar(reinterpret_cast<const char *>(src)) + lane * 16;
    if (is8) {
#pragma unroll
      for (int k = 0; k < N8; ++k) pg_stage16(base + k * 1024, dst + k * 1024);
    } else {
#pragma unroll
      for (int k = 0; k < N16; ++k) pg_stage16(base + k * 1024, dst + k * 1024);
    }
  } else {
    pg_stage_rows<PgStage<D>::BYTES / 1024>(reinterpret_cast<const char *>(src), 0, rows - 1,
                                            PgStage<D>::LG_D + (is8 ? 0 : 1), dst, lane);
  }
}

template <int V>
struct PgBuf {
  static constexpr int value = V;
};

// NB bytes (1, 2, 4, 8 or a multiple of 16, aligned to min(NB, 16)) of LDS as
// 32-bit words; words past them are zero
template <int NB, int NW>
__device__ __forceinline__ void pg_lds_read(const char *p, uint32_t (&w)[NW]) {
  constexpr int N = (NB + 3) / 4;
  static_assert(N <= NW, "chunk words");
#pragma unroll
  for (int e = N; e < NW; ++e) w[e] = 0u;
  if constexpr (NB == 1) {
    w[0] = *reinterpret_cast<const uint8_t *>(p);
  } else if constexpr (NB == 2) {
    w[0] = *reinterpret_cast<const uint16_t *>(p);
  } else if constexpr (NB == 4) {
    w[0] = *reinterpret_cast<const uint32_t *>(p);
  } else if constexpr (NB == 8) {
    const u32x2 x = *reinterpret_cast<const u32x2 *>(p);
    w[0] = x.x;
    w[1] = x.y;
  } else {
    static_assert(NB % 16 == 0, "chunk bytes");
#pragma unroll
    for (int b = 0; b < NB / 16; ++b) {
      const u32x4 x = reinterpret_cast<const u32x4 *>(p)[b];
      w[4 * b] = x.x;
      w[4 * b + 1] = x.y;
      w[4 * b + 2] = x.z;
      w[4 * b + 3] = x.w;
    }
  }
}

// reductions over the four lanes of a head slot (l, l ^ 16, l ^ 32, l ^ 48)
// with the row and half-wave swaps: plain VALU work, no LDS round trip.
// Each step combines a lane's value with its partner's in either order,
// and max and + are commutative, so all four lanes end with the same value.
// (the maximum as one instruction: the values are results of arithmetic,
// never signalling NaNs, so they need no quieting first)
__device__ __forceinline__ float pg_vmax(uint32_t a, uint32_t b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float pg_max4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = pg_vmax(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return pg_vmax(b[0], b[1]);
}
__device__ __forceinline__ float pg_sum4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef __bf16 pg_bf16x8 __attribute__((ext_vector_type(8)));

// the tile's scores before scaling, K in format KF: on the bf16 matrix
// instruction when the query is bf16 and K is bf16 or affine (codes enter
// as the exact bf16 integers c - zp; every product is exact), else on the
// fp32 one with K widened to binary32
// the key operand of the bf16 score product: the lane's K chunk as bf16
// pairs (bf16 K as it is; affine codes c - zp, exact in bf16 as |c - zp| <= 255)
template <int D, int KF, bool ZP = true>
__device__ __forceinline__ void pg_key_bf16(const uint32_t (&w)[D / 4], int32_t kz, uint32_t (&kw)[D / 8]) {
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    if constexpr (KF == SWRT_XF_BF16) {
      kw[i] = w[i];
    } else {
      kw[i] = bf16_pack_hi(pg_elem<KF, ZP>(w, 2 * i, kz), pg_elem<KF, ZP>(w, 2 * i + 1, kz));
    }
  }
}

// the score product on the bf16 matrix instruction (every product exact)
template <int D, typename Q>
__device__ __forceinline__ f32x4 pg_scores_bf16(const uint32_t (&kw)[D / 8], const Q &q) {
  f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int st = 0; st < D / 32; ++st)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(pg_bf16x8, u32x4{kw[4 * st], kw[4 * st + 1], kw[4 * st + 2], kw[4 * st + 3]}),
        __builtin_bit_cast(pg_bf16x8, u32x4{q.b[4 * st], q.b[4 * st + 1], q.b[4 * st + 2], q.b[4 * st + 3]}),
        sc, 0, 0, 0);
  return sc;
}

template <int D, int KF, bool QBF, bool ZP = true>
__device__ __forceinline__ f32x4 pg_scores_words(const uint32_t (&w)[D / 4], const PgQuery<D, QBF> &q,
                                                 int32_t kz) {
  constexpr int KQ = D / 4;
  f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (QBF && KF != SWRT_XF_F32 && KF != SWRT_XF_F16) {
    uint32_t kw[KQ / 2];
    pg_key_bf16<D, KF, ZP>(w, kz, kw);
    sc = pg_scores_bf16<D>(kw, q);
  } else {
#pragma unroll
    for (int e = 0; e < KQ; ++e)
      sc = __builtin_amdgcn_mfma_f32_16x16x4f32(pg_elem<KF>(w, e, kz), q.f(e), sc, 0, 0, 0);
  }
  return sc;
}

// the lane's K chunk read from the staged tile kt
template <int D, int KF>
__device__ __forceinline__ void pg_key_chunk(const char *kt, uint32_t pk, uint32_t qg, uint32_t (&w)[D / 4]) {
  constexpr int NB = D / 4 * pg_bits(KF) / 8;  // at least 2 bytes
  pg_lds_read<NB>(kt + pk * (D * pg_bits(KF) / 8) + qg * NB, w);
}

template <int D, int KF, bool QBF, bool ZP = true>
__device__ __forceinline__ f32x4 pg_tile_scores_t(const char *kt, uint32_t pk, uint32_t qg,
                                                  const PgQuery<D, QBF> &q, int32_t kz) {
  uint32_t w[D / 4];
  pg_key_chunk<D, KF>(kt, pk, qg, w);
  return pg_scores_words<D, KF, QBF, ZP>(w, q, kz);
}

typedef short pg_s16x4 __attribute__((ext_vector_type(4)));

// the tile's weighted values, V in format VF, into the accumulators. Lane
// (j, q) holds rows q + 4 c (c = 0..3) of V, elements MT j .. MT j + MT - 1,
// and the weights of the same rows. bf16 and affine V go through
// v_mfma_f32_16x16x16_bf16 (its four k-slots per lane are those four rows;
// V exact in bf16, the weights as three exact bf16 parts), fp32 and f16 V
// through v_mfma_f32_16x16x4_f32 (one row per instruction).
// the value operand of the bf16 product for output tile m: element m of
// rows 0, 1 and of rows 2, 3 as bf16 pairs (affine codes c - zp, exact in
// bf16 as |c - zp| <= 255)
template <int D, int VF, bool ZP = true>
__device__ __forceinline__ void pg_value_bf16(const uint32_t (&w)[4][D / 16], int32_t vz,
                                              uint32_t (&va)[D / 16][2]) {
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    if constexpr (VF == SWRT_XF_BF16) {
      const uint32_t sel = m % 2 ? 0x07060302u : 0x05040100u;
      va[m][0] = __builtin_amdgcn_perm(w[1][m / 2], w[0][m / 2], sel);
      va[m][1] = __builtin_amdgcn_perm(w[3][m / 2], w[2][m / 2], sel);
    } else {
      va[m][0] = bf16_pack_hi(pg_elem<VF, ZP>(w[0], m, vz), pg_elem<VF, ZP>(w[1], m, vz));
      va[m][1] = bf16_pack_hi(pg_elem<VF, ZP>(w[2], m, vz), pg_elem<VF, ZP>(w[3], m, vz));
    }
  }
}

// the value product on the bf16 matrix instruction, the weights in three
// exact bf16 parts, the small parts first
template <int D>
__device__ __forceinline__ void pg_values_bf16(const uint32_t (&va)[D / 16][2], const float (&pw)[4],
                                               f32x4 (&acc)[D / 16]) {
  uint32_t pb[3][2];
  bf16_split3(pw, pb);
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    const pg_s16x4 a = __builtin_bit_cast(pg_s16x4, u32x2{va[m][0], va[m][1]});
#pragma unroll
    for (int k = 2; k >= 0; --k)
      acc[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          a, __builtin_bit_cast(pg_s16x4, u32x2{pb[k][0], pb[k][1]}), acc[m], 0, 0, 0);
  }
}

template <int D, int VF, bool ZP = true>
__device__ __forceinline__ void pg_values_words(const uint32_t (&w)[4][D / 16], const float (&pw)[4],
                                                int32_t vz, f32x4 (&acc)[D / 16]) {
  constexpr int MT = D / 16;
  if constexpr (VF == SWRT_XF_BF16 || pg_affine(VF)) {
    uint32_t va[MT][2];
    pg_value_bf16<D, VF, ZP>(w, vz, va);
    pg_values_bf16<D>(va, pw, acc);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int m = 0; m < MT; ++m)
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(pg_elem<VF>(w[c], m, vz), pw[c], acc[m], 0, 0, 0);
  }
}

// the lane's four V chunks read from the staged tile vt (a chunk of fewer
// than 8 bits is shifted down from its place in its byte)
template <int D, int VF>
__device__ __forceinline__ void pg_value_chunks(const char *vt, uint32_t j, uint32_t qg,
                                                uint32_t (&w)[4][D / 16]) {
  constexpr int MT = D / 16, BITS = MT * pg_bits(VF), RB = D * pg_bits(VF) / 8;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const char *row = vt + (4 * c + qg) * RB;
    if constexpr (BITS >= 8) {
      pg_lds_read<BITS / 8>(row + j * (BITS / 8), w[c]);
    } else {
      pg_lds_read<1>(row + j * BITS / 8, w[c]);
      w[c][0] >>= (j * BITS) % 8;
    }
  }
}

template <int D, int VF, bool ZP = true>
__device__ __forceinline__ void pg_tile_values_t(const char *vt, uint32_t j, uint32_t qg, const float (&pw)[4],
                                                 int32_t vz, f32x4 (&acc)[D / 16]) {
  uint32_t w[4][D / 16];
  pg_value_chunks<D, VF>(vt, j, qg, w);
  pg_values_words<D, VF, ZP>(w, pw, vz, acc);
}

// the staged formats of 16 bits and fewer but f16 and the last one (the
// switch's default); an fp32 page never reaches these
#define SWRT_PG_NARROW_FORMATS(X) \
  X(SWRT_XF_BF16) X(SWRT_XF_INT8) X(SWRT_XF_UINT8) X(SWRT_XF_INT4) X(SWRT_XF_UINT4) \
  X(SWRT_XF_INT2)

// The page formats a kernel is built for (the set the caller declares): every
// path costs registers and scalar work in the tile loop, so a kernel carries
// only the ones that may occur.
//   kPgLean:   bf16 and int8 pages only (the usual hot and cold formats)
//   kPgNarrow: every staged format but f16
//   kPgWide:   all of them (f16 staged; fp32 read by its own tile code)
constexpr int kPgLean = 0, kPgNarrow = 1, kPgWide = 2;
constexpr uint32_t kPgLeanFormats = (1u << SWRT_XF_BF16) | (1u << SWRT_XF_INT8);

template <int D, bool QBF, int FS>
__device__ __forceinline__ f32x4 pg_tile_scores(int kf, const char *kt, uint32_t pk, uint32_t qg,
                                                const PgQuery<D, QBF> &q, int32_t kz) {
  // the usual page formats first (int8 codes of a zero point 0 without the
  // subtraction), then the rest (uniform in the wave)
  if (kf == SWRT_XF_INT8)
    return kz ? pg_tile_scores_t<D, SWRT_XF_INT8, QBF>(kt, pk, qg, q, kz)
              : pg_tile_scores_t<D, SWRT_XF_INT8, QBF, false>(kt, pk, qg, q, 0);
  if (FS == kPgLean || kf == SWRT_XF_BF16) return pg_tile_scores_t<D, SWRT_XF_BF16, QBF>(kt, pk, qg, q, kz);
  switch (kf) {
#define SWRT_PG_K(F) \
  case F: return pg_tile_scores_t<D, F, QBF>(kt, pk, qg, q, kz);
    SWRT_PG_NARROW_FORMATS(SWRT_PG_K)
#undef SWRT_PG_K
    case SWRT_XF_F16:
      if constexpr (FS == kPgWide) return pg_tile_scores_t<D, SWRT_XF_F16, QBF>(kt, pk, qg, q, kz);
      [[fallthrough]];
    default: return pg_tile_scores_t<D, SWRT_XF_UINT2, QBF>(kt, pk, qg, q, kz);
  }
}

template <int D, int FS>
__device__ __forceinline__ void pg_tile_values(int vf, const char *vt, uint32_t j, uint32_t qg,
                                               const float (&pw)[4], int32_t vz, f32x4 (&acc)[D / 16]) {
  // the usual page formats first (int8 codes of a zero point 0 without the
  // subtraction), then the rest (uniform in the wave)
  if (vf == SWRT_XF_INT8)
    return vz ? pg_tile_values_t<D, SWRT_XF_INT8>(vt, j, qg, pw, vz, acc)
              : pg_tile_values_t<D, SWRT_XF_INT8, false>(vt, j, qg, pw, 0, acc);
  if (FS == kPgLean || vf == SWRT_XF_BF16) return pg_tile_values_t<D, SWRT_XF_BF16>(vt, j, qg, pw, vz, acc);
  switch (vf) {
#define SWRT_PG_V(F) \
  case F: pg_tile_values_t<D, F>(vt, j, qg, pw, vz, acc); break;
    SWRT_PG_NARROW_FORMATS(SWRT_PG_V)
#undef SWRT_PG_V
    case SWRT_XF_F16:
      if constexpr (FS == kPgWide) {
        pg_tile_values_t<D, SWRT_XF_F16>(vt, j, qg, pw, vz, acc);
        break;
      }
      [[fallthrough]];
    default: pg_tile_values_t<D, SWRT_XF_UINT2>(vt, j, qg, pw, vz, acc); break;
  }
}

// Lane l holds head slot j = l % 16 of every accumulator. The score product
// (v_mfma_f32_16x16x4_f32, one dimension per lane and instruction) gives lane
// l the scores of tile rows q + 4 r (q = l / 16) when the key operand carries
// tile row i / 4 + 4 (i % 4) at matrix row i; lane group q covers dimensions
// [q D/4, (q + 1) D/4). The value product's k-th instruction takes rows
// 4 k .. 4 k + 3 of the tile, weights straight from each lane's r = k score,
// and output dimension MT i + m at matrix row i of output tile m
// (MT = D / 16): a lane reads MT consecutive elements of a V row and ends
// holding 4 MT consecutive output dimensions of its head. FS: the page
// formats the kernel is built for (the declared ones; others are refused).
// The bf16 + int8 build for head_dim 64 and a bf16 query fits five waves per
// SIMD (96 registers, no spills; its staging buffers fill a compute unit's
// LDS at five workgroups), one more than its register count would otherwise
// allow.
template <int D, bool QBF, int FS>
__global__ __launch_bounds__(kPgBlock)
__attribute__((amdgpu_waves_per_eu(FS == kPgLean && QBF && D == 64 ? 6 : 1))) void paged_attention_kernel(
    PgAttArgs a) {
  constexpr int KQ = D / 4;   // dimensions per lane of the score product
  constexpr int MT = D / 16;  // output tiles; V elements per lane and row
  using Stage = PgStage<D>;
  // a wave's staging space: the bf16 + int8 tile loop keeps one K buffer and
  // two V buffers, the general one NBUF buffers of K and V
  constexpr bool kLeanLoop = FS == kPgLean && Stage::NBUF == 2;
  constexpr int kWaveStage = kLeanLoop ? 3 * Stage::BYTES : Stage::NBUF * 2 * Stage::BYTES;
  __shared__ __attribute__((aligned(16))) char stage_all[kPgWaves][kWaveStage];
  // the wave index is uniform: everything derived from it (the stream, the
  // layer's pointers) then lives in scalar registers
  const uint32_t lane = threadIdx.x % 64, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const uint32_t j = lane % 16, qg = lane / 16;
  // Workgroups go to the eight XCDs in turn. Each layer's workgroups start at
  // a multiple of 8, so the waves of one stream in every layer run on the
  // same XCD, where layers that share a block table find its ids and
  // descriptors in that XCD's L2.
  const uint32_t layer = blockIdx.x / uint32_t(a.wg_layer);
  const uint32_t item = (blockIdx.x - layer * uint32_t(a.wg_layer)) * kPgWaves + wave;
  if (item >= uint32_t(a.items)) return;
  char *stage = stage_all[wave];
  // an item is (stream, chunk) of the layer: the chunk's query heads are
  // 16 chunk .. 16 chunk + 15 of the group (a group of more than 16 heads is
  // split over consecutive items, whose waves read the same pages)
  const uint32_t chunk = item % uint32_t(a.chunks), str = item / uint32_t(a.chunks);
  const uint32_t g = str % uint32_t(a.Hkv), b = str / uint32_t(a.Hkv);
  const PgLayer &P = a.L[layer];
  const char *const arena = P.arena;
  const int G = a.Hq / a.Hkv;
  const int hs = int(16 * chunk + j);  // this lane's head within the group
  const bool head = hs < G;
  const int64_t s = int64_t(b) * a.Hkv + g;

  // query operand: head slot j's dimensions of lane group qg
  PgQuery<D, QBF> q;
  {
    float qf[KQ];
    const uint64_t qrow = uint64_t(b) * a.Hq + g * G + (head ? hs : 0);
    const int qes = a.q_type == SWRT_XF_F32 ? 4 : 2;
    const char *qp = P.q + qrow * uint64_t(D) * qes;
    pg_load_decode<KQ>(a.q_type, qp, qg * KQ, 0, qf);
#pragma unroll
    for (int k = 0; k < KQ; ++k) qf[k] = head ? qf[k] : 0.0f;
    q.set(qf);
  }

  float m = -INFINITY, l_sum = 0.0f;
  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  int64_t ptr0, ptr1;
  bool ok = pg_stream_range(P, s, ptr0, ptr1);
  if (ok && ptr1 > ptr0) {
    // Pages are taken 64 at a time from the last one back: lane l reads the
    // whole descriptor of page top - l (ids, then descriptors, one load each
    // for the group) and checks it, joined to its successor by
    // start + length == the successor's start. The last page fixes T and the
    // window's first token r0; a group's pages from its lane 0 down to the
    // first starting at or before r0 are visible. Pages the window does not
    // reach are neither decoded nor checked beyond their id and start.
    const int32_t pk = (j >> 2) + 4 * (j & 3);  // tile row of this lane's key operand
    int64_t T = -1, r0 = 0, next_start = 0;
    bool done = false;
    for (int64_t top = ptr1 - 1; ok && !done; top -= 64) {
      const int64_t k = top - lane;
      const bool in = k >= ptr0;
      int32_t id = 0;
      if (in) id = P.page_ids[k];
      bool good = !in || (id >= 0 && id < P.n_pages);
      swrt_page d = {};
      if (in && good) {
        d = P.pages[id];
        good = pg_page_ok(d, D, P.arena_bytes) && (k != ptr0 || d.start == 0) &&
               ((a.formats >> d.k_format) & (a.formats >> d.v_format) & 1u);
      }
      const int64_t end = d.start + d.length;
      const uint32_t elo = uint32_t(end), ehi = uint32_t(uint64_t(end) >> 32);
      const uint32_t slo = uint32_t(d.start), shi = uint32_t(uint64_t(d.start) >> 32);
      if (T < 0) {  // the first group: its lane 0 holds the last page
        T = int64_t((uint64_t(uint32_t(__builtin_amdgcn_readlane(int(ehi), 0))) << 32) |
                    uint32_t(__builtin_amdgcn_readlane(int(elo), 0)));
        r0 = a.left_window < 0 ? 0 : (T - 1 - a.left_window > 0 ? T - 1 - a.left_window : 0);
        next_start = T;
      }
      const int64_t succ = int64_t((uint64_t(uint32_t(__shfl_up(int(shi), 1))) << 32) |
                                   uint32_t(__shfl_up(int(slo), 1)));
      if (in && good) good = end == (lane == 0 ? next_start : succ);
      const uint64_t hits = __builtin_amdgcn_ballot_w64(in && good && d.start <= r0);
      const uint64_t ins = __builtin_amdgcn_ballot_w64(in);
      const int h = hits ? __builtin_ctzll(hits) : 63;  // the last lane to take
      const uint64_t mine = h == 63 ? ~0ull : (2ull << h) - 1;
      if (__builtin_amdgcn_ballot_w64(in && !good) & mine) {
        ok = false;
        break;
      }
      if (!hits && (ins >> 63) == 0) {  // out of pages with none starting at or before r0
        ok = false;
        break;
      }
      done = hits != 0;
      const int n_in = hits ? h + 1 : 64;
      next_start = int64_t((uint64_t(uint32_t(__builtin_amdgcn_readlane(int(shi), n_in - 1))) << 32) |
                           uint32_t(__builtin_amdgcn_readlane(int(slo), n_in - 1)));
      // Each lane's page packed for the tile loop: both formats, the row the
      // window starts at in it, both zero points (each fits 16 bits).
      const int32_t p_fmt = d.k_format | (d.v_format << 8);
      const int32_t p_first = r0 > d.start ? int32_t(min(r0 - d.start, int64_t(d.length))) : 0;
      const int32_t p_zp = (d.k_zero_point & 0xFFFF) | (d.v_zero_point << 16);
      // page l's fields, uniform
      auto field = [&](int32_t x, int l) { return __builtin_amdgcn_readlane(x, l); };
      auto field64 = [&](int64_t x, int l) {
        return int64_t((uint64_t(uint32_t(field(int32_t(uint64_t(x) >> 32), l))) << 32) |
                       uint32_t(field(int32_t(x), l)));
      };
      // The tile's weights from its scores (rows from `rows` on masked): the
      // online maximum and sum move on, and the accumulators with them.
      auto weigh = [&](const f32x4 &sc, float ks, float vs, int32_t rows, float (&pw)[4]) {
#pragma clang fp contract(off)
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = sc[r] * ks;
        if (rows < 16) {  // a partial tile (uniform): rows past the page's last masked
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = int32_t(qg) + 4 * r < rows ? x[r] : -INFINITY;
        }
        float bm = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) bm = fmaxf(bm, x[r]);
        bm = pg_max4(bm);
        // the reference maximum moves only when a tile's exceeds it by more
        // than 2^8 (log2 units); a single visible token still weighs 1
        const bool move = bm > m + 8.0f;
        const float mn = move ? bm : m;
        if (__builtin_amdgcn_ballot_w64(move && m != -INFINITY)) {
          const float f = move ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;
          l_sum *= f;
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[t] *= f;
        }
        const float ms = mn == -INFINITY ? 0.0f : mn;  // no finite score yet: every weight 0
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float w = __builtin_amdgcn_exp2f(x[r] - ms);
          l_sum += w;
          pw[r] = w * vs;  // an affine page's V scale rides on the weight
        }
        m = mn;
      };
      if constexpr (kLeanLoop) {
        // Every page bf16 or int8 (K and V apart). Per page, once for the
        // group: the payload addresses at the window's first row, the rows
        // from there, the formats, the scales (K's with the softmax scale).
        const bool k8 = d.k_format == SWRT_XF_INT8, v8 = d.v_format == SWRT_XF_INT8;
        const int64_t abase = int64_t(reinterpret_cast<uintptr_t>(arena));
        const int64_t p_k = abase + d.k_offset + (int64_t(p_first) << (Stage::LG_D + (k8 ? 0 : 1)));
        const int64_t p_v = abase + d.v_offset + (int64_t(p_first) << (Stage::LG_D + (v8 ? 0 : 1)));
        const int32_t p_rows = d.length - p_first;
        const int32_t p_kind = (k8 ? 1 : 0) | (v8 ? 2 : 0);
        const float p_ks = k8 ? d.k_scale * a.scale_log2 : a.scale_log2;
        const float p_vs = v8 ? d.v_scale : 1.0f;
        struct PgLean {
          int64_t k, v;  // this tile's first K and V rows
          int32_t rows, kind, zp;
          float ks, vs;
        };
        auto lean_of = [&](int l) {
          PgLean c;
          c.k = field64(p_k, l);
          c.v = field64(p_v, l);
          c.rows = field(p_rows, l);
          c.kind = field(p_kind, l);
          c.zp = field(p_zp, l);
          c.ks = __int_as_float(field(__float_as_int(p_ks), l));
          c.vs = __int_as_float(field(__float_as_int(p_vs), l));
          return c;
        };
        // K has one buffer: a tile's K chunks are read out at its start and
        // the next tile's K rows staged right after. V has two: the next
        // tile's V rows are staged as a tile starts.
        auto stage_k = [&](const PgLean &c) { pg_stage_lean<D>(c.k, c.rows, c.kind & 1, stage, lane); };
        auto stage_v = [&](const PgLean &c, int buf) {
          pg_stage_lean<D>(c.v, c.rows, c.kind & 2, stage + (1 + buf) * Stage::BYTES, lane);
        };
        // One tile from buffer BUF (the next one staged first, into the other
        // buffer); false after the group's last tile. Two calls an
        // iteration, so that the buffers alternate at compile time.
        int l = n_in - 1;
        auto tile = [&](auto bufc, const PgLean &c, PgLean &n) {
          constexpr int BUF = decltype(bufc)::value;
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this tile's rows have landed
          // the next tile: the page's next 16 rows, or the next page's first
          // (read from any lane when there is none)
          if (c.rows > 16) {
            n = c;
            n.k = c.k + ((c.kind & 1) ? 16 * D : 32 * D);
            n.v = c.v + ((c.kind & 2) ? 16 * D : 32 * D);
            n.rows = c.rows - 16;
          } else {
            --l;
            n = lean_of(l & 63);
          }
          const bool more = l >= 0;
          if (more) stage_v(n, BUF ^ 1);
          const char *vt = stage + (1 + BUF) * Stage::BYTES;
          const int32_t kz = int16_t(c.zp), vz = c.zp >> 16;
          // this tile's K chunk, then the next tile's K rows into the buffer
          uint32_t w[D / 4];
          if (!(c.kind & 1))
            pg_key_chunk<D, SWRT_XF_BF16>(stage, pk, qg, w);
          else
            pg_key_chunk<D, SWRT_XF_INT8>(stage, pk, qg, w);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read out before the refill
          if (more) stage_k(n);
          float pw[4];
          if constexpr (QBF) {
            // the operands decoded per format, one chain of products for all
            uint32_t kw[D / 8];
            if (!(c.kind & 1))
              pg_key_bf16<D, SWRT_XF_BF16>(w, 0, kw);
            else if (kz)
              pg_key_bf16<D, SWRT_XF_INT8>(w, kz, kw);
            else
              pg_key_bf16<D, SWRT_XF_INT8, false>(w, 0, kw);
            weigh(pg_scores_bf16<D>(kw, q), c.ks, c.vs, c.rows, pw);
            uint32_t va[D / 16][2];
            if (!(c.kind & 2)) {
              uint32_t vw[4][D / 16];
              pg_value_chunks<D, SWRT_XF_BF16>(vt, j, qg, vw);
              pg_value_bf16<D, SWRT_XF_BF16>(vw, 0, va);
            } else {
              uint32_t vw[4][D / 16];
              pg_value_chunks<D, SWRT_XF_INT8>(vt, j, qg, vw);
              if (vz)
                pg_value_bf16<D, SWRT_XF_INT8>(vw, vz, va);
              else
                pg_value_bf16<D, SWRT_XF_INT8, false>(vw, 0, va);
            }
            pg_values_bf16<D>(va, pw, acc);
          } else {
            f32x4 sc;
            if (!(c.kind & 1))
              sc = pg_scores_words<D, SWRT_XF_BF16, QBF>(w, q, 0);
            else if (kz)
              sc = pg_scores_words<D, SWRT_XF_INT8, QBF>(w, q, kz);
            else
              sc = pg_scores_words<D, SWRT_XF_INT8, QBF, false>(w, q, 0);
            weigh(sc, c.ks, c.vs, c.rows, pw);
            if (!(c.kind & 2))
              pg_tile_values_t<D, SWRT_XF_BF16>(vt, j, qg, pw, 0, acc);
            else if (vz)
              pg_tile_values_t<D, SWRT_XF_INT8>(vt, j, qg, pw, vz, acc);
            else
              pg_tile_values_t<D, SWRT_XF_INT8, false>(vt, j, qg, pw, 0, acc);
          }
          return more;
        };
        PgLean c0 = lean_of(l), c1 = c0;
        stage_v(c0, 0);
        stage_k(c0);
        while (true) {
          if (!tile(PgBuf<0>(), c0, c1)) break;
          if (!tile(PgBuf<1>(), c1, c0)) break;
        }
      } else {
        // what the tile code needs of page l, uniform
        struct PgCur {
          int kf, vf;
          int32_t len, kz, vz;
          float ks, vs;
        };
        auto cur_of = [&](int l) {
          PgCur c;
          const int32_t fmt = field(p_fmt, l), zp = field(p_zp, l);
          c.kf = fmt & 0xFF;
          c.vf = fmt >> 8;
          c.len = field(d.length, l);
          const bool ka = pg_affine(c.kf), va = pg_affine(c.vf);
          c.ks = ka ? __int_as_float(field(__float_as_int(d.k_scale), l)) * a.scale_log2 : a.scale_log2;
          c.vs = va ? __int_as_float(field(__float_as_int(d.v_scale), l)) : 1.0f;
          c.kz = ka ? int32_t(int16_t(zp)) : 0;
          c.vz = va ? zp >> 16 : 0;
          return c;
        };
        // Stage rows [i, i + 16) of page l's K and V payloads (an fp32 payload
        // is read by its tile code instead) into buffer buf.
        auto stage_tile = [&](int l, int32_t i, int buf, const PgCur &c) {
          char *dst = stage + buf * (2 * Stage::BYTES);
          const int32_t lim = c.len - 1 - i;
          constexpr int NMAX = Stage::BYTES / 1024;
          // log2 row bytes
          const int klg = FS == kPgLean ? Stage::LG_D + (c.kf == SWRT_XF_INT8 ? 0 : 1)
                                        : Stage::LG_D + int((kPgLogBits >> (4 * c.kf)) & 15) - 3;
          const int vlg = FS == kPgLean ? Stage::LG_D + (c.vf == SWRT_XF_INT8 ? 0 : 1)
                                        : Stage::LG_D + int((kPgLogBits >> (4 * c.vf)) & 15) - 3;
          if (c.kf != SWRT_XF_F32) pg_stage_rows<NMAX>(arena + field64(d.k_offset, l), i, lim, klg, dst, lane);
          if (c.vf != SWRT_XF_F32)
            pg_stage_rows<NMAX>(arena + field64(d.v_offset, l), i, lim, vlg, dst + Stage::BYTES, lane);
        };
        // The group's visible pages in token order: lanes n_in - 1 .. 0. With
        // two buffers the next tile is staged before this one is computed.
        int l = n_in - 1;
        int32_t i = field(p_first, l);
        // One tile of page l from buffer BUF, rows [i, i + 16): the next
        // tile's page fields into cn and its rows into the other buffer
        // first (two buffers), or into the same buffer after (one); false
        // after the group's last tile.
        auto step = [&](auto bufc, const PgCur &c, PgCur &cn) {
          constexpr int BUF = decltype(bufc)::value;
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this tile's rows have landed
          // the tile after this one
          int ln = l;
          int32_t in_ = i + 16;
          cn = c;
          if (in_ >= c.len) {
            ln = l - 1;
            in_ = 0;
            if (ln >= 0) {
              cn = cur_of(ln);
              in_ = field(p_first, ln);
            }
          }
          if constexpr (Stage::NBUF == 2) {
            if (ln >= 0) stage_tile(ln, in_, BUF ^ 1, cn);
          }
          const char *kt = stage + BUF * (2 * Stage::BYTES), *vt = kt + Stage::BYTES;
          // this tile: page l's formats and scales
          const int kf = c.kf, vf = c.vf;
          const int32_t len = c.len;
          const int32_t kz = c.kz, vz = c.vz;
          f32x4 sc;
          if (FS == kPgWide && kf == SWRT_XF_F32) {  // not staged
            uint32_t w[KQ];
            pg_load_raw<KQ * 4>(arena + field64(d.k_offset, l) +
                                    int64_t(min(i + pk, len - 1)) * (4 * D) + int64_t(qg) * (4 * KQ),
                                w);
            sc = pg_scores_words<D, SWRT_XF_F32, QBF>(w, q, 0);
          } else {
            sc = pg_tile_scores<D, QBF, FS>(kf, kt, pk, qg, q, kz);
          }
          float pw[4];
          weigh(sc, c.ks, c.vs, len - i, pw);
          if (FS == kPgWide && vf == SWRT_XF_F32) {  // not staged
            uint32_t w[4][MT];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              pg_load_raw<MT * 4>(arena + field64(d.v_offset, l) +
                                      int64_t(min(i + 4 * r + int32_t(qg), len - 1)) * (4 * D) +
                                      int64_t(j) * (4 * MT),
                                  w[r]);
            pg_values_words<D, SWRT_XF_F32>(w, pw, 0, acc);
          } else {
            pg_tile_values<D, FS>(vf, vt, j, qg, pw, vz, acc);
          }
          if (ln < 0) return false;
          if constexpr (Stage::NBUF == 1) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this tile read out before the refill
            stage_tile(ln, in_, 0, cn);
          }
          l = ln;
          i = in_;
          return true;
        };
        PgCur c0 = cur_of(l), c1 = c0;
        stage_tile(l, i, 0, c0);
        if constexpr (Stage::NBUF == 2) {  // two tiles an iteration: the buffers alternate
          while (true) {
            if (!step(PgBuf<0>(), c0, c1)) break;
            if (!step(PgBuf<1>(), c1, c0)) break;
          }
        } else {
          while (true) {
            if (!step(PgBuf<0>(), c0, c1)) break;
            c0 = c1;
          }
        }
      }
    }
  }
  if (!ok) {  // no output for this stream's heads
    if (a.flags && lane == 0) atomicOr(a.flags, SWRT_FLAG_BAD_PAGES);
    return;
  }
  l_sum = pg_sum4(l_sum);
  if (!head) return;
  const float inv = l_sum > 0.0f ? 1.0f / l_sum : 0.0f;  // no visible token: zeros
  float y[4 * MT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) y[MT * r + t] = acc[t][r] * inv;
  const uint64_t orow = uint64_t(b) * a.Hq + g * G + hs;
  if (a.out_type == SWRT_XF_F32) {
    u32x4 *dst = reinterpret_cast<u32x4 *>(P.out + (orow * D + 4 * MT * qg) * 4);
#pragma unroll
    for (int c = 0; c < MT; ++c)
      dst[c] = u32x4{__float_as_uint(y[4 * c]), __float_as_uint(y[4 * c + 1]),
                     __float_as_uint(y[4 * c + 2]), __float_as_uint(y[4 * c + 3])};
  } else {
    uint32_t h[2 * MT];
#pragma unroll
    for (int e = 0; e < 2 * MT; ++e) {
      const uint32_t lo = a.out_type == SWRT_XF_BF16 ? xf_bf16(y[2 * e]) : xf_f16(y[2 * e]);
      const uint32_t hi = a.out_type == SWRT_XF_BF16 ? xf_bf16(y[2 * e + 1]) : xf_f16(y[2 * e + 1]);
      h[e] = lo | (hi << 16);
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(P.out + (orow * D + 4 * MT * qg) * 2);
#pragma unroll
    for (int c = 0; c < MT / 2; ++c) dst[c] = u32x4{h[4 * c], h[4 * c + 1], h[4 * c + 2], h[4 * c + 3]};
  }
}

// ---------------------------------------------------------------------------
// encoding eight consecutive elements (conversion and append)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int32_t pg_code(float y, float scale, int32_t zp, int32_t lo, int32_t hi) {
  if (y != y) return zp;
  float q = __builtin_rintf(y / scale) + float(zp);  // ties to even
  q = fminf(fmaxf(q, float(lo)), float(hi));
  return int32_t(q);
}

template <int FMT>
__device__ __forceinline__ void pg_store8_t(char *dst, const float (&y)[8], float scale, int32_t zp) {
  if constexpr (FMT == SWRT_XF_F32) {
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = y[e] != y[e] ? 0x7FC00000u : __float_as_uint(y[e]);
    __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, pg_gw(reinterpret_cast<u32x4 *>(dst)));
    __builtin_nontemporal_store(u32x4{w[4], w[5], w[6], w[7]}, pg_gw(reinterpret_cast<u32x4 *>(dst) + 1));
  } else if constexpr (FMT == SWRT_XF_F16 || FMT == SWRT_XF_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = FMT == SWRT_XF_BF16 ? xf_bf16(y[2 * e]) : xf_f16(y[2 * e]);
      const uint32_t hi = FMT == SWRT_XF_BF16 ? xf_bf16(y[2 * e + 1]) : xf_f16(y[2 * e + 1]);
      w[e] = lo | (hi << 16);
    }
    __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, pg_gw(reinterpret_cast<u32x4 *>(dst)));
  } else {
    constexpr int B = pg_bits(FMT);
    uint64_t packed = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t c = uint32_t(pg_code(y[e], scale, zp, pg_lo(FMT), pg_hi(FMT))) & ((1u << B) - 1u);
      packed |= uint64_t(c) << (e * B);
    }
    if constexpr (B == 8) {
      __builtin_nontemporal_store(u32x2{uint32_t(packed), uint32_t(packed >> 32)},
                                  pg_gw(reinterpret_cast<u32x2 *>(dst)));
    } else if constexpr (B == 4) {
      __builtin_nontemporal_store(uint32_t(packed), pg_gw(reinterpret_cast<uint32_t *>(dst)));
    } else {
      __builtin_nontemporal_store(uint16_t(packed), pg_gw(reinterpret_cast<uint16_t *>(dst)));
    }
  }
}

__device__ __forceinline__ void pg_store8(int fmt, char *dst, const float (&y)[8], float scale,
                                          int32_t zp) {
  switch (fmt) {
    case SWRT_XF_F32: pg_store8_t<SWRT_XF_F32>(dst, y, scale, zp); break;
    case SWRT_XF_F16: pg_store8_t<SWRT_XF_F16>(dst, y, scale, zp); break;
    case SWRT_XF_BF16: pg_store8_t<SWRT_XF_BF16>(dst, y, scale, zp); break;
    case SWRT_XF_INT8: pg_store8_t<SWRT_XF_INT8>(dst, y, scale, zp); break;
    case SWRT_XF_UINT8: pg_store8_t<SWRT_XF_UINT8>(dst, y, scale, zp); break;
    case SWRT_XF_INT4: pg_store8_t<SWRT_XF_INT4>(dst, y, scale, zp); break;
    case SWRT_XF_UINT4: pg_store8_t<SWRT_XF_UINT4>(dst, y, scale, zp); break;
    case SWRT_XF_INT2: pg_store8_t<SWRT_XF_INT2>(dst, y, scale, zp); break;
    default: pg_store8_t<SWRT_XF_UINT2>(dst, y, scale, zp); break;
  }
}

// eight elements of a page row decoded in binary32: dense as is, affine as
// fl((c - zp) * scale), one rounding
__device__ __forceinline__ void pg_value8(int fmt, const char *row, uint32_t first, float scale,
                                          int32_t zp, float (&y)[8]) {
  pg_load_decode<8>(fmt, row, first, pg_affine(fmt) ? zp : 0, y);
  if (pg_affine(fmt)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = y[e] * scale;
  }
}

// ---------------------------------------------------------------------------
// conversion of selected pages
// ---------------------------------------------------------------------------
struct PgConvArgs {
  char *arena;
  int64_t arena_bytes;
  const swrt_page *pages_in;
  swrt_page *pages_out;
  int64_t n_pages;
  const int32_t *blocks;
  int64_t n_blocks;
  const int64_t *dst;
  int64_t free_begin, free_end;
  uint32_t *flags;
  int32_t fmt[2];
  float scale[2];  // 1 for a dense target
  int32_t zp[2];   // 0 for a dense target
  int32_t D;
};

__device__ __forceinline__ bool pg_overlap(int64_t a0, int64_t n0, int64_t a1, int64_t n1) {
  return n0 > 0 && n1 > 0 && a0 < a1 + n1 && a1 < a0 + n0;
}

// every page, and every selected block with its destinations
__global__ __launch_bounds__(kPgBlock) void paged_validate_kernel(PgConvArgs a) {
  const int64_t n = a.n_pages + a.n_blocks;
  bool bad = false;
  for (int64_t x = int64_t(blockIdx.x) * kPgBlock + threadIdx.x; x < n;
       x += int64_t(gridDim.x) * kPgBlock) {
    if (x < a.n_pages) {
      const swrt_page p = a.pages_in[x];
      const int64_t fr = a.free_end - a.free_begin;
      bad |= !pg_page_ok(p, a.D, a.arena_bytes) ||
             pg_overlap(a.free_begin, fr, p.k_offset, p.capacity * pg_row_bytes(p.k_format, a.D)) ||
             pg_overlap(a.free_begin, fr, p.v_offset, p.capacity * pg_row_bytes(p.v_format, a.D));
    } else {
      const int64_t i = x - a.n_pages;
      const int32_t id = a.blocks[i];
      if (id < 0 || id >= a.n_pages || (i > 0 && id <= a.blocks[i - 1])) {
        bad = true;
        continue;
      }
      const int64_t cap = a.pages_in[id].capacity;
      int64_t prev_end = a.free_begin;  // where this block's K may start
      if (i > 0) {
        const int32_t pid = a.blocks[i - 1];
        if (pid < 0 || pid >= a.n_pages) {
          bad = true;
          continue;
        }
        prev_end = a.dst[2 * i - 1] + a.pages_in[pid].capacity * pg_row_bytes(a.fmt[1], a.D);
      }
      const int64_t kb = cap * pg_row_bytes(a.fmt[0], a.D), vb = cap * pg_row_bytes(a.fmt[1], a.D);
      const int64_t dk = a.dst[2 * i], dv = a.dst[2 * i + 1];
      bad |= cap < 1 || dk < prev_end || (dk & 15) != 0 || kb > a.free_end - dk ||
             dv < dk + kb || (dv & 15) != 0 || vb > a.free_end - dv;
    }
  }
  if (bad) atomicOr(a.flags, SWRT_FLAG_BAD_PAGES);
}

// one wave per (selected block, K or V): every row of the capacity, eight
// elements per lane step; rows past the page's length are logical zeros
__global__ __launch_bounds__(64) void paged_convert_kernel(PgConvArgs a) {
  if (__atomic_load_n(a.flags, __ATOMIC_RELAXED) & SWRT_FLAG_BAD_PAGES) return;
  const int64_t i = blockIdx.x / 2;
  const int t = blockIdx.x % 2;
  const swrt_page p = pg_read(a.pages_in, a.blocks[i]);
  const int sf = t ? p.v_format : p.k_format;
  const float ss = t ? p.v_scale : p.k_scale;
  const int32_t sz = t ? p.v_zero_point : p.k_zero_point;
  const int df = a.fmt[t];
  const int64_t srow = pg_row_bytes(sf, a.D), drow = pg_row_bytes(df, a.D);
  const char *src = a.arena + (t ? p.v_offset : p.k_offset);
  char *dst = a.arena + a.dst[2 * i + t];
  const int32_t per_row = a.D / 8;
  const int64_t n = int64_t(p.capacity) * per_row;
  for (int64_t o = threadIdx.x; o < n; o += 64) {
    const int64_t r = o / per_row;
    const uint32_t e0 = uint32_t(o % per_row) * 8;
    float y[8];
    if (r < p.length) {
      pg_value8(sf, src + r * srow, e0, ss, sz, y);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = 0.0f;
    }
    pg_store8(df, dst + r * drow + int64_t(e0) * pg_bits(df) / 8, y, a.scale[t], a.zp[t]);
  }
}

// the selected descriptors with their new storage, written in place
__device__ __forceinline__ void pg_retarget(const PgConvArgs &a, swrt_page &p, int64_t i) {
  p.k_format = a.fmt[0];
  p.v_format = a.fmt[1];
  p.k_scale = a.scale[0];
  p.v_scale = a.scale[1];
  p.k_zero_point = a.zp[0];
  p.v_zero_point = a.zp[1];
  p.k_offset = a.dst[2 * i];
  p.v_offset = a.dst[2 * i + 1];
}

__global__ __launch_bounds__(kPgBlock) void paged_publish_selected_kernel(PgConvArgs a) {
  if (__atomic_load_n(a.flags, __ATOMIC_RELAXED) & SWRT_FLAG_BAD_PAGES) return;
  for (int64_t i = int64_t(blockIdx.x) * kPgBlock + threadIdx.x; i < a.n_blocks;
       i += int64_t(gridDim.x) * kPgBlock) {
    swrt_page p = a.pages_in[a.blocks[i]];
    pg_retarget(a, p, i);
    a.pages_out[a.blocks[i]] = p;
  }
}

// every descriptor to a separate pages_out, the selected ones with their new
// storage
__global__ __launch_bounds__(kPgBlock) void paged_publish_kernel(PgConvArgs a) {
  if (__atomic_load_n(a.flags, __ATOMIC_RELAXED) & SWRT_FLAG_BAD_PAGES) return;
  for (int64_t x = int64_t(blockIdx.x) * kPgBlock + threadIdx.x; x < a.n_pages;
       x += int64_t(gridDim.x) * kPgBlock) {
    swrt_page p = a.pages_in[x];
    // blocks are ascending: binary search for x
    int64_t lo = 0, hi = a.n_blocks;
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (a.blocks[mid] < x)
        lo = mid + 1;
      else
        hi = mid;
    }
    if (lo < a.n_blocks && a.blocks[lo] == x) pg_retarget(a, p, lo);
    a.pages_out[x] = p;
  }
}

// ---------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------
struct PgAppArgs {
  PgLayer L[kMaxLayers];
  const char *k_new[kMaxLayers];
  const char *v_new[kMaxLayers];
  int32_t table[kMaxLayers];  // layers whose block tables are distinct
  uint32_t *flags;
  int32_t n_streams, n_tables, D, new_type, items;
};

// the page stream s's token goes to, and whether it can take it
__device__ __forceinline__ uint32_t pg_append_target(const PgLayer &P, int64_t s, int D, int32_t &id,
                                                     swrt_page &p) {
  int64_t ptr0, ptr1;
  if (!pg_stream_range(P, s, ptr0, ptr1) || ptr1 == ptr0) return SWRT_FLAG_BAD_PAGES;
  id = __builtin_amdgcn_readfirstlane(P.page_ids[ptr1 - 1]);
  if (id < 0 || id >= P.n_pages) return SWRT_FLAG_BAD_PAGES;
  p = pg_read(P.pages, id);
  if (!pg_page_ok(p, D, P.arena_bytes)) return SWRT_FLAG_BAD_PAGES;
  return p.length == p.capacity ? SWRT_FLAG_PAGE_FULL : 0u;
}

// one wave per (layer, stream): the new K and V rows, encoded, as row
// `length` of the stream's last page
__global__ __launch_bounds__(kPgBlock) void paged_append_rows_kernel(PgAppArgs a) {
  const uint32_t lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const uint32_t item = blockIdx.x * kPgWaves + wave;
  if (item >= uint32_t(a.items)) return;
  const int64_t s = item % uint32_t(a.n_streams);
  const uint32_t layer = item / uint32_t(a.n_streams);
  const PgLayer &P = a.L[layer];
  int32_t id;
  swrt_page p;
  const uint32_t bad = pg_append_target(P, s, a.D, id, p);
  if (bad) {
    if (a.flags && lane == 0) atomicOr(a.flags, bad);
    return;
  }
  const int nes = a.new_type == SWRT_XF_F32 ? 4 : 2;
  for (int t = 0; t < 2; ++t) {
    const int fmt = t ? p.v_format : p.k_format;
    const float sc = t ? p.v_scale : p.k_scale;
    const int32_t zp = t ? p.v_zero_point : p.k_zero_point;
    const char *in = (t ? a.v_new[layer] : a.k_new[layer]) + s * a.D * nes;
    char *row = const_cast<char *>(P.arena) + (t ? p.v_offset : p.k_offset) +
                int64_t(p.length) * pg_row_bytes(fmt, a.D);
    for (int e0 = int(lane) * 8; e0 < a.D; e0 += 64 * 8) {
      float y[8];
      pg_load_decode<8>(a.new_type, in, uint32_t(e0), 0, y);
      pg_store8(fmt, row + int64_t(e0) * pg_bits(fmt) / 8, y, sc, zp);
    }
  }
}

// after every layer's rows: each distinct block table's appended pages grow
// by one row (the same checks decide, on the same descriptors)
__global__ __launch_bounds__(kPgBlock) void paged_append_commit_kernel(PgAppArgs a) {
  const int64_t x = int64_t(blockIdx.x) * kPgBlock + threadIdx.x;
  if (x >= int64_t(a.n_tables) * a.n_streams) return;
  const PgLayer &P = a.L[a.table[x / a.n_streams]];
  const int64_t s = x % a.n_streams;
  int64_t ptr0, ptr1;
  if (!pg_stream_range<false>(P, s, ptr0, ptr1) || ptr1 == ptr0) return;
  const int32_t id = P.page_ids[ptr1 - 1];
  if (id < 0 || id >= P.n_pages) return;
  swrt_page *pg = const_cast<swrt_page *>(P.pages) + id;
  if (pg_page_ok(*pg, a.D, P.arena_bytes) && pg->length < pg->capacity) pg->length += 1;
}

// ---------------------------------------------------------------------------
// sealed append: one new block per stream
// ---------------------------------------------------------------------------
struct PgSealArgs {
  PgLayer L[kMaxLayers];
  const char *k_new[kMaxLayers];
  const char *v_new[kMaxLayers];
  int8_t order[kMaxLayers];          // layers, each table's consecutive
  int8_t group_begin[kMaxLayers + 1];
  uint32_t *flags;
  int64_t first_id, free_begin, kb, vb;
  int32_t fmt[2];
  float scale[2];  // 1 for a dense format
  int32_t zp[2];   // 0 for a dense format
  int32_t n_groups, n_streams, S, D, new_type, items;
};

// One wave per (block table, stream): check the stream's last block (the
// only descriptor read), encode the S new rows of every layer sharing the
// table into the stream's room of the free region, then write the new
// block's descriptor and take the stream's next slot. Streams touch
// disjoint slots, descriptors and payload room, and no wave writes a
// descriptor another reads (the last block's id may not be a new one), so
// the waves need no ordering among themselves.
__global__ __launch_bounds__(kPgBlock) void paged_append_sealed_kernel(PgSealArgs a) {
  const uint32_t lane = threadIdx.x % 64, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const uint32_t item = blockIdx.x * kPgWaves + wave;
  if (item >= uint32_t(a.items)) return;
  const int64_t s = item % uint32_t(a.n_streams);
  const int grp = int(item / uint32_t(a.n_streams));
  const PgLayer &T0 = a.L[a.order[a.group_begin[grp]]];  // the table's fields
  int64_t p0, p1;
  uint32_t bad = 0;
  int64_t T = 0;
  if (!pg_stream_range(T0, s, p0, p1)) {
    bad = SWRT_FLAG_BAD_PAGES;
  } else if (p1 == p0 + T0.page_stride) {
    bad = SWRT_FLAG_PAGE_FULL;  // no free slot for the new block
  } else if (p1 > p0) {
    const int32_t last = __builtin_amdgcn_readfirstlane(T0.page_ids[p1 - 1]);
    if (last < 0 || last >= T0.n_pages || (last >= a.first_id && last < a.first_id + a.n_streams)) {
      bad = SWRT_FLAG_BAD_PAGES;
    } else {
      const swrt_page d = pg_read(T0.pages, last);
      if (!pg_page_ok(d, a.D, T0.arena_bytes) || d.start + d.length > INT64_MAX - a.S)
        bad = SWRT_FLAG_BAD_PAGES;
      else
        T = d.start + d.length;
    }
  }
  if (bad) {
    if (a.flags && lane == 0) atomicOr(a.flags, bad);
    return;
  }
  const int64_t koff = a.free_begin + s * (a.kb + a.vb), voff = koff + a.kb;
  const int nes = a.new_type == SWRT_XF_F32 ? 4 : 2;
  const int32_t per_row = a.D / 8;
  const int64_t n8 = int64_t(a.S) * per_row;  // eight-element groups per tensor
  for (int i = a.group_begin[grp]; i < a.group_begin[grp + 1]; ++i) {
    const int layer = a.order[i];
    char *arena = const_cast<char *>(a.L[layer].arena);
    for (int t = 0; t < 2; ++t) {
      const int fmt = a.fmt[t];
      const char *in = (t ? a.v_new[layer] : a.k_new[layer]) + s * int64_t(a.S) * a.D * nes;
      char *dst = arena + (t ? voff : koff);
      for (int64_t o = lane; o < n8; o += 64) {
        const int64_t r = o / per_row;
        const uint32_t e0 = uint32_t(o - r * per_row) * 8;
        float y[8];
        pg_load_decode<8>(a.new_type, in + r * a.D * nes, e0, 0, y);
        pg_store8(fmt, dst + (r * a.D + e0) * pg_bits(fmt) / 8, y, a.scale[t], a.zp[t]);
      }
    }
  }
  if (lane == 0) {
    const int64_t id = a.first_id + s;
    swrt_page np = {};
    np.start = T;
    np.length = a.S;
    np.capacity = a.S;
    np.k_offset = koff;
    np.v_offset = voff;
    np.k_format = a.fmt[0];
    np.v_format = a.fmt[1];
    np.k_scale = a.scale[0];
    np.v_scale = a.scale[1];
    np.k_zero_point = a.zp[0];
    np.v_zero_point = a.zp[1];
    const_cast<swrt_page *>(T0.pages)[id] = np;
    const_cast<int32_t *>(T0.page_ids)[p1] = int32_t(id);
    T0.page_count[s] = int32_t(p1 - p0 + 1);
  }
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------
bool pg_q_type_ok(int t) { return t == SWRT_XF_F32 || t == SWRT_XF_F16 || t == SWRT_XF_BF16; }

// the per-layer fields the kernels read, checked for what the host can see
int pg_layers(int n_layers, const swrt_paged_layer *layers, PgLayer *out, bool attention,
              int64_t n_streams) {
  for (int l = 0; l < n_layers; ++l) {
    const swrt_paged_layer &x = layers[l];
    if (!x.arena || !x.pages || (!x.page_ptr && !x.page_count) || (x.n_ids > 0 && !x.page_ids))
      return SWRT_E_INVALID_ARG;
    if (x.arena_bytes < 0 || x.arena_bytes % 16 || x.n_pages < 0 || x.n_ids < 0 ||
        x.n_pages > INT32_MAX || (x.page_count && x.page_stride < 1))
      return SWRT_E_INVALID_ARG;
    if (addr_of(x.arena) % 16 || addr_of(x.pages) % 8 || addr_of(x.page_ptr) % 4 ||
        addr_of(x.page_ids) % 4 || addr_of(x.page_count) % 4)
      return SWRT_E_INVALID_ARG;
    if (attention && (!x.q || !x.out || addr_of(x.q) % 16 || addr_of(x.out) % 16))
      return SWRT_E_INVALID_ARG;
    out[l] = PgLayer{static_cast<const char *>(x.q), static_cast<char *>(x.out),
                     static_cast<const char *>(x.arena), x.arena_bytes, x.pages, x.n_pages,
                     x.page_count ? nullptr : x.page_ptr, x.page_ids, x.n_ids, x.page_count,
                     x.page_count ? x.page_stride : 0};
    (void)n_streams;
  }
  return SWRT_OK;
}

// the block table's read range of a layer: page_ptr (compressed rows) or
// page_count (slotted rows)
Range pg_table_range(const swrt_paged_layer &x, int64_t n_streams, bool written) {
  return x.page_count ? range(x.page_count, uint64_t(n_streams) * 4, written)
                      : range(x.page_ptr, uint64_t(n_streams + 1) * 4, written);
}

// Layers that share a block table: either all of pages, the table form and
// page_ids, or none of them. group[l] = the first layer with l's table.
int pg_groups(int n_layers, const swrt_paged_layer *layers, int32_t *group) {
  for (int l = 0; l < n_layers; ++l) {
    group[l] = l;
    const swrt_paged_layer &y = layers[l];
    for (int e = 0; e < l; ++e) {
      const swrt_paged_layer &x = layers[e];
      const int same = int(x.pages == y.pages) + int(x.page_ids == y.page_ids) +
                       int(x.page_ptr == y.page_ptr && x.page_count == y.page_count);
      if (same == 0) continue;
      if (same != 3 || x.n_pages != y.n_pages || x.n_ids != y.n_ids ||
          x.page_stride != y.page_stride)
        return SWRT_E_INVALID_ARG;  // partly shared
      group[l] = group[e];
      break;
    }
  }
  return SWRT_OK;
}

}  // namespace
}  // namespace swrt

using namespace swrt;

extern "C" int swrt_paged_attention(int n_layers, const swrt_paged_layer *layers,
                                    int64_t left_window, int batch, int q_heads, int kv_heads,
                                    int head_dim, float scale, int q_type, int out_type,
                                    uint32_t page_formats, uint32_t *d_flags, void *stream) {
  if (n_layers < 0 || n_layers > kMaxLayers || batch < 0 || q_heads < 0 || kv_heads < 1)
    return SWRT_E_INVALID_ARG;
  if (!pg_q_type_ok(q_type) || !pg_q_type_ok(out_type) || q_heads % kv_heads)
    return SWRT_E_INVALID_ARG;
  if (!(scale == scale) || scale > 3.4028235e38f || scale < -3.4028235e38f) return SWRT_E_INVALID_ARG;
  constexpr uint32_t kAllFormats = 0x3FEu;  // bits 1 .. 9: F32 .. UINT2
  if (page_formats & ~kAllFormats) return SWRT_E_INVALID_ARG;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256)
    return SWRT_E_UNSUPPORTED;
  if (n_layers == 0 || batch == 0 || q_heads == 0) return SWRT_OK;
  if (!layers || addr_of(d_flags) % 4) return SWRT_E_INVALID_ARG;
  const int chunks = int((int64_t(q_heads / kv_heads) + 15) / 16);  // items per stream
  int64_t items;
  if (!mul_ok(int64_t(n_layers) * batch, int64_t(kv_heads) * chunks, &items) ||
      items >= (int64_t(1) << 31))
    return SWRT_E_UNSUPPORTED;
  PgAttArgs a;
  const int st = pg_layers(n_layers, layers, a.L, true, int64_t(batch) * kv_heads);
  if (st != SWRT_OK) return st;
  // outputs must not overlap any input of the call
  Range ranges[6 * kMaxLayers + 1];
  int nr = 0;
  const int64_t qes = q_type == SWRT_XF_F32 ? 4 : 2, oes = out_type == SWRT_XF_F32 ? 4 : 2;
  int64_t rows, q_bytes, o_bytes;  // elements of q and out; head_dim <= 256
  if (!mul_ok(int64_t(batch) * q_heads, head_dim, &rows) || !mul_ok(rows, qes, &q_bytes) ||
      !mul_ok(rows, oes, &o_bytes))
    return SWRT_E_UNSUPPORTED;
  for (int l = 0; l < n_layers; ++l) {
    const swrt_paged_layer &x = layers[l];
    ranges[nr++] = range(x.q, uint64_t(q_bytes), false);
    ranges[nr++] = range(x.out, uint64_t(o_bytes), true);
    ranges[nr++] = range(x.arena, uint64_t(x.arena_bytes), false);
    ranges[nr++] = range(x.pages, uint64_t(x.n_pages) * sizeof(swrt_page), false);
    ranges[nr++] = pg_table_range(x, int64_t(batch) * kv_heads, false);
    ranges[nr++] = range(x.page_ids, uint64_t(x.n_ids) * 4, false);
  }
  ranges[nr++] = range(d_flags, 4, true);
  if (written_overlap(ranges, nr)) return SWRT_E_INVALID_ARG;
  a.flags = d_flags;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.left_window = left_window;
  a.B = batch;
  a.Hq = q_heads;
  a.Hkv = kv_heads;
  a.items = batch * kv_heads * chunks;
  a.wg_layer = int32_t((int64_t(a.items) + 8 * kPgWaves - 1) / (8 * kPgWaves) * 8);
  a.chunks = chunks;
  a.q_type = q_type;
  a.out_type = out_type;
  a.formats = page_formats ? page_formats : kAllFormats;
  // the build for the declared formats: bf16 and int8 only, or without fp32
  // and f16, or all (fewer paths, fewer registers and less scalar work)
  const int fs = (a.formats & ~kPgLeanFormats) == 0 ? kPgLean
                 : (a.formats & ((1u << SWRT_XF_F32) | (1u << SWRT_XF_F16))) == 0 ? kPgNarrow
                                                                                   : kPgWide;
  static_assert(sizeof(PgAttArgs) <= 4096, "kernel arguments exceed 4 KiB");
  const dim3 grid(uint32_t(n_layers) * uint32_t(a.wg_layer));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool qbf = q_type == SWRT_XF_BF16;
#define SWRT_PG_LAUNCH_FS(DD, QB, FS) \
  hipLaunchKernelGGL((paged_attention_kernel<DD, QB, FS>), grid, dim3(kPgBlock), 0, s, a);
#define SWRT_PG_LAUNCH_Q(DD, QB)                                 \
  if (fs == kPgLean) SWRT_PG_LAUNCH_FS(DD, QB, kPgLean)          \
  else if (fs == kPgNarrow) SWRT_PG_LAUNCH_FS(DD, QB, kPgNarrow) \
  else SWRT_PG_LAUNCH_FS(DD, QB, kPgWide)
#define SWRT_PG_LAUNCH(DD)          \
  if (qbf) SWRT_PG_LAUNCH_Q(DD, true) \
  else SWRT_PG_LAUNCH_Q(DD, false)
  switch (head_dim) {
    case 32: SWRT_PG_LAUNCH(32) break;
    case 64: SWRT_PG_LAUNCH(64) break;
    case 128: SWRT_PG_LAUNCH(128) break;
    default: SWRT_PG_LAUNCH(256) break;
  }
#undef SWRT_PG_LAUNCH
#undef SWRT_PG_LAUNCH_Q
#undef SWRT_PG_LAUNCH_FS
  return launch_status();
}

extern "C" int swrt_paged_quantize(void *arena, int64_t arena_bytes, const swrt_page *pages_in,
                                   int64_t n_pages, const int32_t *blocks, int64_t n_blocks,
                                   const int64_t *dst_offsets, int64_t free_begin,
                                   int64_t free_end, swrt_page *pages_out, int k_format,
                                   float k_scale, int32_t k_zero_point, int v_format,
                                   float v_scale, int32_t v_zero_point, int head_dim,
                                   uint32_t *d_flags, void *stream) {
  if (n_pages < 0 || n_blocks < 0 || arena_bytes < 0 || head_dim < 16 || head_dim % 16 ||
      head_dim > 4096)
    return SWRT_E_INVALID_ARG;
  if (!pg_format_ok(k_format, k_scale, k_zero_point) || !pg_format_ok(v_format, v_scale, v_zero_point))
    return SWRT_E_INVALID_ARG;
  if (free_begin < 0 || free_end < free_begin || free_end > arena_bytes) return SWRT_E_INVALID_ARG;
  if (!d_flags || addr_of(d_flags) % 4) return SWRT_E_INVALID_ARG;
  if (n_pages > INT32_MAX || n_blocks > n_pages) return SWRT_E_INVALID_ARG;
  if (n_pages == 0) return SWRT_OK;
  if (!arena || !pages_in || !pages_out || (n_blocks > 0 && (!blocks || !dst_offsets)))
    return SWRT_E_INVALID_ARG;
  if (addr_of(arena) % 16 || addr_of(pages_in) % 8 || addr_of(pages_out) % 8 ||
      addr_of(blocks) % 4 || addr_of(dst_offsets) % 8)
    return SWRT_E_INVALID_ARG;
  // descriptors and the flag word are written: they overlap no input other
  // than pages_out == pages_in
  Range ranges[6];
  int nr = 0;
  ranges[nr++] = range(arena, uint64_t(arena_bytes), true);
  if (pages_out != pages_in) ranges[nr++] = range(pages_in, uint64_t(n_pages) * sizeof(swrt_page), false);
  ranges[nr++] = range(pages_out, uint64_t(n_pages) * sizeof(swrt_page), true);
  ranges[nr++] = range(blocks, uint64_t(n_blocks) * 4, false);
  ranges[nr++] = range(dst_offsets, uint64_t(n_blocks) * 16, false);
  ranges[nr++] = range(d_flags, 4, true);
  if (written_overlap(ranges, nr)) return SWRT_E_INVALID_ARG;
  PgConvArgs a;
  a.arena = static_cast<char *>(arena);
  a.arena_bytes = arena_bytes;
  a.pages_in = pages_in;
  a.pages_out = pages_out;
  a.n_pages = n_pages;
  a.blocks = blocks;
  a.n_blocks = n_blocks;
  a.dst = dst_offsets;
  a.free_begin = free_begin;
  a.free_end = free_end;
  a.flags = d_flags;
  a.fmt[0] = k_format;
  a.fmt[1] = v_format;
  a.scale[0] = pg_affine(k_format) ? k_scale : 1.0f;
  a.scale[1] = pg_affine(v_format) ? v_scale : 1.0f;
  a.zp[0] = pg_affine(k_format) ? k_zero_point : 0;
  a.zp[1] = pg_affine(v_format) ? v_zero_point : 0;
  a.D = head_dim;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nv = n_pages + n_blocks;
  const uint32_t gv = uint32_t(std::min<int64_t>((nv + kPgBlock - 1) / kPgBlock, 4096));
  hipLaunchKernelGGL(paged_validate_kernel, dim3(gv), dim3(kPgBlock), 0, s, a);
  int st = launch_status();
  if (st != SWRT_OK) return st;
  if (n_blocks > 0) {
    if (n_blocks > (int64_t(1) << 30)) return SWRT_E_UNSUPPORTED;
    hipLaunchKernelGGL(paged_convert_kernel, dim3(uint32_t(2 * n_blocks)), dim3(64), 0, s, a);
    st = launch_status();
    if (st != SWRT_OK) return st;
  }
  if (pages_out == pages_in) {  // in place: only the selected descriptors change
    if (n_blocks == 0) return SWRT_OK;
    const uint32_t gb = uint32_t(std::min<int64_t>((n_blocks + kPgBlock - 1) / kPgBlock, 4096));
    hipLaunchKernelGGL(paged_publish_selected_kernel, dim3(gb), dim3(kPgBlock), 0, s, a);
    return launch_status();
  }
  const uint32_t gp = uint32_t(std::min<int64_t>((n_pages + kPgBlock - 1) / kPgBlock, 4096));
  hipLaunchKernelGGL(paged_publish_kernel, dim3(gp), dim3(kPgBlock), 0, s, a);
  return launch_status();
}

extern "C" int swrt_paged_append_open(int n_layers, const swrt_paged_layer *layers,
                                      const void *const *k_new, const void *const *v_new,
                                      int new_type, int n_streams, int head_dim, uint32_t *d_flags,
                                      void *stream) {
  if (n_layers < 0 || n_layers > kMaxLayers || n_streams < 0 || !pg_q_type_ok(new_type))
    return SWRT_E_INVALID_ARG;
  if (head_dim < 16 || head_dim % 16 || head_dim > 4096) return SWRT_E_INVALID_ARG;
  if (n_layers == 0 || n_streams == 0) return SWRT_OK;
  if (!layers || !k_new || !v_new || addr_of(d_flags) % 4) return SWRT_E_INVALID_ARG;
  if (uint64_t(n_layers) * n_streams >= (uint64_t(1) << 31)) return SWRT_E_UNSUPPORTED;
  PgAppArgs a;
  int st = pg_layers(n_layers, layers, a.L, false, n_streams);
  if (st != SWRT_OK) return st;
  // the lengths of each distinct block table grow once
  int32_t group[kMaxLayers];
  if ((st = pg_groups(n_layers, layers, group)) != SWRT_OK) return st;
  a.n_tables = 0;
  for (int l = 0; l < n_layers; ++l)
    if (group[l] == l) a.table[a.n_tables++] = l;
  const int64_t nes = new_type == SWRT_XF_F32 ? 4 : 2;
  Range ranges[7 * kMaxLayers + 1];
  int nr = 0;
  for (int l = 0; l < n_layers; ++l) {
    const swrt_paged_layer &x = layers[l];
    if (!k_new[l] || !v_new[l] || addr_of(k_new[l]) % 16 || addr_of(v_new[l]) % 16)
      return SWRT_E_INVALID_ARG;
    a.k_new[l] = static_cast<const char *>(k_new[l]);
    a.v_new[l] = static_cast<const char *>(v_new[l]);
    ranges[nr++] = range(x.arena, uint64_t(x.arena_bytes), true);
    ranges[nr++] = range(k_new[l], uint64_t(n_streams) * head_dim * nes, false);
    ranges[nr++] = range(v_new[l], uint64_t(n_streams) * head_dim * nes, false);
  }
  for (int t = 0; t < a.n_tables; ++t) {  // each distinct table once
    const swrt_paged_layer &x = layers[a.table[t]];
    ranges[nr++] = range(x.pages, uint64_t(x.n_pages) * sizeof(swrt_page), true);
    ranges[nr++] = pg_table_range(x, n_streams, false);
    ranges[nr++] = range(x.page_ids, uint64_t(x.n_ids) * 4, false);
  }
  ranges[nr++] = range(d_flags, 4, true);
  if (written_overlap(ranges, nr)) return SWRT_E_INVALID_ARG;
  a.flags = d_flags;
  a.n_streams = n_streams;
  a.D = head_dim;
  a.new_type = new_type;
  a.items = n_layers * n_streams;
  static_assert(sizeof(PgAppArgs) <= 4096, "kernel arguments exceed 4 KiB");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(paged_append_rows_kernel, dim3((uint32_t(a.items) + kPgWaves - 1) / kPgWaves),
                     dim3(kPgBlock), 0, s, a);
  const int st2 = launch_status();
  if (st2 != SWRT_OK) return st2;
  const int64_t nc = int64_t(a.n_tables) * n_streams;
  hipLaunchKernelGGL(paged_append_commit_kernel, dim3(uint32_t((nc + kPgBlock - 1) / kPgBlock)),
                     dim3(kPgBlock), 0, s, a);
  return launch_status();
}

extern "C" int swrt_paged_append(int n_layers, const swrt_paged_layer *layers,
                                 const void *const *k_new, const void *const *v_new, int new_type,
                                 int n_streams, int seq_len, int head_dim, int64_t first_id,
                                 int64_t free_begin, int64_t free_end, int k_format, float k_scale,
                                 int32_t k_zero_point, int v_format, float v_scale,
                                 int32_t v_zero_point, uint32_t *d_flags, void *stream) {
  // what the definition itself rejects
  if (n_layers < 0 || n_layers > kMaxLayers || n_streams < 0 || seq_len < 1 ||
      !pg_q_type_ok(new_type) || head_dim < 1)
    return SWRT_E_INVALID_ARG;
  if (!pg_format_ok(k_format, k_scale, k_zero_point) || !pg_format_ok(v_format, v_scale, v_zero_point))
    return SWRT_E_INVALID_ARG;
  // the library's layout rule: 16-byte blocks of payload
  if (head_dim < 16 || head_dim % 16 || head_dim > 4096) return SWRT_E_UNSUPPORTED;
  const int64_t kb = int64_t(seq_len) * head_dim * pg_bits(k_format) / 8;
  const int64_t vb = int64_t(seq_len) * head_dim * pg_bits(v_format) / 8;
  if (n_layers == 0) return SWRT_OK;
  if (!layers || addr_of(d_flags) % 4) return SWRT_E_INVALID_ARG;
  for (int l = 0; l < n_layers; ++l) {
    const swrt_paged_layer &x = layers[l];
    if (!x.page_count || x.page_stride < 1) return SWRT_E_INVALID_ARG;  // slotted rows only
    if (x.n_pages < 0 || first_id < 0 || first_id > x.n_pages - n_streams)
      return SWRT_E_INVALID_ARG;
    if (free_begin < 0 || free_end < free_begin || free_end > x.arena_bytes ||
        (n_streams > 0 && kb + vb > (free_end - free_begin) / n_streams))
      return SWRT_E_INVALID_ARG;
    if (n_streams > x.n_ids / x.page_stride) return SWRT_E_INVALID_ARG;
  }
  if (free_begin % 16 || kb % 16 || vb % 16) return SWRT_E_UNSUPPORTED;
  if (n_streams == 0) return SWRT_OK;
  if (!k_new || !v_new) return SWRT_E_INVALID_ARG;
  if (uint64_t(n_layers) * n_streams >= (uint64_t(1) << 31) ||
      uint64_t(seq_len) * head_dim >= (uint64_t(1) << 31))
    return SWRT_E_UNSUPPORTED;
  PgSealArgs a;
  int st = pg_layers(n_layers, layers, a.L, false, n_streams);
  if (st != SWRT_OK) return st;
  int32_t group[kMaxLayers];
  if ((st = pg_groups(n_layers, layers, group)) != SWRT_OK) return st;
  // layers ordered so that each table's layers are consecutive
  a.n_groups = 0;
  int n = 0;
  for (int l = 0; l < n_layers; ++l) {
    if (group[l] != l) continue;
    a.group_begin[a.n_groups++] = n;
    for (int e = l; e < n_layers; ++e)
      if (group[e] == l) {
        if (layers[e].arena_bytes != layers[l].arena_bytes) return SWRT_E_INVALID_ARG;
        a.order[n++] = e;
      }
  }
  a.group_begin[a.n_groups] = n;
  const int64_t nes = new_type == SWRT_XF_F32 ? 4 : 2;
  const uint64_t new_bytes = uint64_t(n_streams) * seq_len * head_dim * nes;
  Range ranges[7 * kMaxLayers + 1];
  int nr = 0;
  for (int l = 0; l < n_layers; ++l) {
    const swrt_paged_layer &x = layers[l];
    if (!k_new[l] || !v_new[l] || addr_of(k_new[l]) % 16 || addr_of(v_new[l]) % 16)
      return SWRT_E_INVALID_ARG;
    a.k_new[l] = static_cast<const char *>(k_new[l]);
    a.v_new[l] = static_cast<const char *>(v_new[l]);
    ranges[nr++] = range(x.arena, uint64_t(x.arena_bytes), true);
    ranges[nr++] = range(k_new[l], new_bytes, false);
    ranges[nr++] = range(v_new[l], new_bytes, false);
  }
  for (int g = 0; g < a.n_groups; ++g) {  // each distinct table once
    const swrt_paged_layer &x = layers[a.order[a.group_begin[g]]];
    ranges[nr++] = range(x.pages, uint64_t(x.n_pages) * sizeof(swrt_page), true);
    ranges[nr++] = range(x.page_count, uint64_t(n_streams) * 4, true);
    ranges[nr++] = range(x.page_ids, uint64_t(x.n_ids) * 4, true);
  }
  ranges[nr++] = range(d_flags, 4, true);
  if (written_overlap(ranges, nr)) return SWRT_E_INVALID_ARG;
  a.flags = d_flags;
  a.n_streams = n_streams;
  a.S = seq_len;
  a.D = head_dim;
  a.new_type = new_type;
  a.first_id = first_id;
  a.free_begin = free_begin;
  a.kb = kb;
  a.vb = vb;
  a.fmt[0] = k_format;
  a.fmt[1] = v_format;
  a.scale[0] = pg_affine(k_format) ? k_scale : 1.0f;
  a.scale[1] = pg_affine(v_format) ? v_scale : 1.0f;
  a.zp[0] = pg_affine(k_format) ? k_zero_point : 0;
  a.zp[1] = pg_affine(v_format) ? v_zero_point : 0;
  a.items = a.n_groups * n_streams;
  static_assert(sizeof(PgSealArgs) <= 4096, "kernel arguments exceed 4 KiB");
  hipLaunchKernelGGL(paged_append_sealed_kernel, dim3((uint32_t(a.items) + kPgWaves - 1) / kPgWaves),
                     dim3(kPgBlock), 0, static_cast<hipStream_t>(stream), a);
  return launch_status();
}
