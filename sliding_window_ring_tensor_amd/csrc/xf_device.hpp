// xf_device.hpp -- the row transform of a fused append.
//
// On its way into the cache a new K or V row (f32, f16 or bf16 elements) is
// read as float; K turns by RoPE at its absolute position (onnxruntime pull
// request "GQA support sliding_window_cache", "Summary of Changes": the append
// uses the cache-relative offset, RoPE the absolute position, bounded by the
// tables' own length and not by the capacity); then every element is written
// in the cache's type: f32, f16 or bf16 rounded to nearest even, an affine
// INT8 / UINT8 code rounded half to even and saturated (onnx-light how-to
// "Persistent input/output feedback", section "Optional heterogeneous paged
// KV"), or an OCP FP8 E4M3 code of y / scale (nearest even, saturating at
// +-448). Scales and zero points are the tensor's scalars or, per channel,
// entry h * head_dim + e of [kv_heads, head_dim] tables (the pull request's
// per-channel shape (kv_num_heads, 1, head_size) with the singleton dropped).
//
// Each pair (x0, x1) -- elements (j, j + rotary_dim/2), or (2j, 2j+1) when
// interleaved -- turns by the angle of table row pos, column j:
//   x0' = x0 c - x1 s,  x1' = x1 c + x0 s,
// each product and each sum one binary32 operation rounded to nearest even
// (no fused multiply-add), so the rounded element and the quantized code are
// decided by fixed arithmetic. NaN becomes the positive canonical quiet NaN
// of a float type (its sign and payload after arithmetic are not fixed), or
// the zero point of an integer code.
//
// A lane produces one VEC-byte word of the output row at a time: the
// VEC / out_bytes elements it covers, their rotation partners and table
// entries are read with plain (cached) loads; rows are small and the
// partners and tables are shared between lanes.
#pragma once

#include "swrt_device.hpp"

namespace swrt {

struct RowXf {
  const float *cos, *sin;  // [max_pos, half] binary32; null: no rotation
  int64_t max_pos;
  int32_t half;            // rotary_dim / 2
  int32_t interleaved;
  int32_t in_type, out_type;    // SWRT_XF_*
  int32_t in_bytes, out_bytes;  // element sizes
  float scale[2];               // K, V (integer and fp8 codes)
  int32_t zero[2];
  int32_t lo, hi;               // code range
  const float *cs[2];           // per-channel scales [heads, d] (K, V), or null
  const int32_t *cz[2];         // per-channel zero points [heads, d], or null
  int32_t d;                    // elements per row: the tables' row length
  int32_t heads;                // rows of the tables (TensorScatter: prefix index mod heads)
};

// any per-channel table (a uniform test on the kernel arguments)
__device__ __forceinline__ bool xf_channels(const RowXf &x) {
  return x.cs[0] || x.cs[1] || x.cz[0] || x.cz[1];
}

// the scale and zero point of element e of a row of KV head h, tensor t.
// The per-tensor scalars are taken as register values (readfirstlane of a
// kernel-uniform value) before the table select: a select between a table
// element and a kernel-argument field would be folded into one load through a
// pointer that may address the arguments, and the compiler then copies the
// whole argument block to scratch memory.
__device__ __forceinline__ void xf_params(const RowXf &x, int t, uint32_t h, uint32_t e, float &sc,
                                          int32_t &zp) {
  const float *cs = t ? x.cs[1] : x.cs[0];
  const int32_t *cz = t ? x.cz[1] : x.cz[0];
  const float s0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x.scale[0])));
  const float s1 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x.scale[1])));
  const int32_t z0 = __builtin_amdgcn_readfirstlane(x.zero[0]);
  const int32_t z1 = __builtin_amdgcn_readfirstlane(x.zero[1]);
  const uint32_t k = h * uint32_t(x.d) + e;
  // the default first, a table entry loaded over it: the path without a table
  // writes no register that a load of the other path may still be filling
  // (such a write would wait for every load in flight)
  sc = t ? s1 : s0;
  zp = t ? z1 : z0;
  if (cs) sc = cs[k];
  if (cz) zp = cz[k];
}

// the same for the N consecutive elements [e0, e0 + N) of one row: one test
// of the table pointers for all of them, the entries loaded side by side
template <int N>
__device__ __forceinline__ void xf_params_n(const RowXf &x, int t, uint32_t h, uint32_t e0,
                                            float (&sc)[N], int32_t (&zp)[N]) {
  const float *cs = t ? x.cs[1] : x.cs[0];
  const int32_t *cz = t ? x.cz[1] : x.cz[0];
  const float s0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x.scale[0])));
  const float s1 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x.scale[1])));
  const int32_t z0 = __builtin_amdgcn_readfirstlane(x.zero[0]);
  const int32_t z1 = __builtin_amdgcn_readfirstlane(x.zero[1]);
  const uint32_t k0 = h * uint32_t(x.d) + e0;
#pragma unroll
  for (int k = 0; k < N; ++k) sc[k] = t ? s1 : s0, zp[k] = t ? z1 : z0;
  if (cs) {
#pragma unroll
    for (int k = 0; k < N; ++k) sc[k] = cs[k0 + k];
  }
  if (cz) {
#pragma unroll
    for (int k = 0; k < N; ++k) zp[k] = cz[k0 + k];
  }
}

// positions [p0, p0 + n) all have table rows (always, without rotation)
__device__ __forceinline__ bool xf_positions_ok(const RowXf &x, int64_t p0, int64_t n) {
  return !x.cos || (p0 >= 0 && p0 <= x.max_pos - n);
}

// binary32 -> bf16 bits, round to nearest even (a carry into the exponent is
// the correct next value, infinity included)
__device__ __forceinline__ uint16_t xf_bf16(float f) {
  if (f != f) return 0x7FC0;
  const uint32_t u = __float_as_uint(f);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t xf_f16(float f) {
  if (f != f) return 0x7E00;
  return __builtin_bit_cast(uint16_t, _Float16(f));  // hardware conversion, nearest even
}

// A NaN quotient (a NaN y, or a per-channel scale that makes y / scale NaN)
// takes the zero point, itself saturated into the code range (a per-channel
// zero point is data the host never sees)
__device__ __forceinline__ int32_t xf_code_of(const RowXf &x, float scale, int32_t zero, float y) {
  const float r = y / scale;
  if (r != r) return min(max(zero, x.lo), x.hi);
  float q = __builtin_rintf(r) + float(zero);
  q = fminf(fmaxf(q, float(x.lo)), float(x.hi));
  return int32_t(q);
}

// OCP FP8 E4M3 (float8e4m3fn) bits of a binary32 value: nearest even; finite
// values past 448 and infinities saturate to +-448 (0x7E / 0xFE), NaN is 0x7F.
// Exponent bias 7, three fraction bits; below 2^-6 the value counts units of
// 2^-9 (subnormals; eight units is the smallest normal, the same bits).
__device__ __forceinline__ uint8_t xf_fp8(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7F;                        // NaN
  if (a >= 0x43E00000u) return uint8_t(sign | 0x7Eu);      // >= 448 (and inf)
  if (a < 0x3C800000u) {                                   // < 2^-6: units of 2^-9
    const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scaling
    return uint8_t(sign | uint32_t(q));
  }
  // normal: keep 3 fraction bits, ties to even (a carry moves the exponent)
  const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
  return uint8_t(sign | (r - (120u << 3)));  // rebias 127 -> 7
}

// one output byte of an integer or fp8 target
__device__ __forceinline__ uint8_t xf_byte(const RowXf &x, float sc, int32_t zp, float y) {
  if (x.out_type == SWRT_XF_FP8_E4M3) return xf_fp8(y / sc);
  return uint8_t(xf_code_of(x, sc, zp, y));  // two's complement bits for INT8
}

// the input element e of a row as float, the input type fixed at compile time
template <int IN>
__device__ __forceinline__ uint32_t xf_raw_t(const char *row, uint32_t e) {
  if constexpr (IN == SWRT_XF_F32)
    return reinterpret_cast<const uint32_t *>(row)[e];
  else
    return uint32_t(reinterpret_cast<const uint16_t *>(row)[e]);
}

template <int IN>
__device__ __forceinline__ float xf_decode_t(uint32_t r) {
  if constexpr (IN == SWRT_XF_F32)
    return __uint_as_float(r);
  else if constexpr (IN == SWRT_XF_BF16)
    return __uint_as_float(r << 16);
  else
    return float(__builtin_bit_cast(_Float16, uint16_t(r)));
}

// element e < rotary_dim: is it the first of its pair, its table column j and
// its partner pe
__device__ __forceinline__ void xf_pair(const RowXf &x, uint32_t e, bool &first, uint32_t &j,
                                        uint32_t &pe) {
  const uint32_t h = uint32_t(x.half);
  first = x.interleaved ? (e & 1u) == 0 : e < h;
  j = x.interleaved ? e >> 1 : (first ? e : e - h);
  pe = x.interleaved ? (e ^ 1u) : (first ? e + h : e - h);
}

// one output element from its raw input, its partner's and its table entries
template <int IN>
__device__ __forceinline__ float xf_rotate(const RowXf &x, bool rot, uint32_t e, uint32_t xr,
                                           uint32_t pr, float c, float s) {
#pragma clang fp contract(off)
  float v = xf_decode_t<IN>(xr);
  if (rot && e < uint32_t(2 * x.half)) {
    bool first;
    uint32_t j, pe;
    xf_pair(x, e, first, j, pe);
    const float vc = v * c, ps = xf_decode_t<IN>(pr) * s;
    v = first ? vc - ps : vc + ps;
  }
  return v;
}

template <int VEC, int IN, int OB, bool ROT>
__device__ __forceinline__ typename Word<VEC>::T xf_word_of(const RowXf &x, int t, uint32_t h,
                                                            const char *row, const float *cr,
                                                            const float *sr, uint32_t i) {
  using W = typename Word<VEC>::T;
  constexpr int N = VEC / OB;  // elements in the word
  uint8_t b[VEC] = {};
  if constexpr (N >= 1) {
    // every load first (straight-line), then the arithmetic
    uint32_t xr[N], pr[N];
    float c[N], s[N];
    float sc[N];
    int32_t zp[N];
    if constexpr (OB == 1) xf_params_n<N>(x, t, h, i * N, sc, zp);
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const uint32_t e = i * N + k;
      xr[k] = xf_raw_t<IN>(row, e);
      pr[k] = 0;
      c[k] = s[k] = 0.0f;
      if constexpr (ROT) {
        bool first;
        uint32_t j, pe;
        xf_pair(x, min(e, uint32_t(2 * x.half) - 1), first, j, pe);
        pr[k] = xf_raw_t<IN>(row, pe);
        c[k] = cr[j];
        s[k] = sr[j];
      }
    }
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const float v = xf_rotate<IN>(x, ROT, i * N + k, xr[k], pr[k], c[k], s[k]);
      if constexpr (OB == 4) {
        const uint32_t u = v != v ? 0x7FC00000u : __float_as_uint(v);
        __builtin_memcpy(b + 4 * k, &u, 4);
      } else if constexpr (OB == 2) {
        const uint16_t h = x.out_type == SWRT_XF_BF16 ? xf_bf16(v) : xf_f16(v);
        __builtin_memcpy(b + 2 * k, &h, 2);
      } else {
        b[k] = xf_byte(x, sc[k], zp[k], v);
      }
    }
  }
  W w;
  __builtin_memcpy(&w, b, VEC);
  return w;
}

template <int VEC, int IN>
__device__ __forceinline__ typename Word<VEC>::T xf_word_in(const RowXf &x, int t, uint32_t h,
                                                            const char *row, int64_t pos,
                                                            uint32_t i) {
  if (t == 0 && x.cos) {
    const float *cr = x.cos + pos * x.half, *sr = x.sin + pos * x.half;
    if (x.out_bytes == 1) return xf_word_of<VEC, IN, 1, true>(x, t, h, row, cr, sr, i);
    if (x.out_bytes == 2) return xf_word_of<VEC, IN, 2, true>(x, t, h, row, cr, sr, i);
    return xf_word_of<VEC, IN, 4, true>(x, t, h, row, cr, sr, i);
  }
  if (x.out_bytes == 1) return xf_word_of<VEC, IN, 1, false>(x, t, h, row, nullptr, nullptr, i);
  if (x.out_bytes == 2) return xf_word_of<VEC, IN, 2, false>(x, t, h, row, nullptr, nullptr, i);
  return xf_word_of<VEC, IN, 4, false>(x, t, h, row, nullptr, nullptr, i);
}

// Word i (VEC bytes of out_type elements) of the transform of `row` of KV head
// h, tensor t (0 = K, rotated when tables are given; 1 = V) at absolute
// position pos. The cache's element alignment makes VEC a multiple of
// out_bytes.
template <int VEC>
__device__ __forceinline__ typename Word<VEC>::T xf_word(const RowXf &x, int t, uint32_t h,
                                                         const char *row, int64_t pos, uint32_t i) {
  if (x.in_type == SWRT_XF_F32) return xf_word_in<VEC, SWRT_XF_F32>(x, t, h, row, pos, i);
  if (x.in_type == SWRT_XF_BF16) return xf_word_in<VEC, SWRT_XF_BF16>(x, t, h, row, pos, i);
  return xf_word_in<VEC, SWRT_XF_F16>(x, t, h, row, pos, i);
}

// ---------------------------------------------------------------------------
// The appended row of an in-place windowed step, spread over the slice's
// lanes: element e belongs to lane e mod n (n lanes, at most kXfLaneElems
// elements each). Its raw input bits, its partner's and its table entries are
// loaded before the shift's loads and turned into cache elements after the
// shift's barrier, so their latency overlaps the shift and each lane's
// arithmetic stays a few elements long. Lanes past the row load its last
// element and store nothing.
// ---------------------------------------------------------------------------
constexpr int kXfLaneElems = 8;

// M: the most elements a lane holds. The registers of all M stay allocated
// for the whole kernel, so kernels whose rows always fit their lanes (one
// element each) take M = 1 and keep their occupancy.
template <int M = kXfLaneElems>
struct XfLanes {
  uint32_t x[M], p[M];  // raw bits of the element and its partner
  float c[M], s[M];     // its table entries (rotated K only)
  float scale[M];       // its scale and zero point (byte targets)
  int32_t zero[M];
};

// Make the loaded values live here: called after the shift's loads are
// issued and before its barrier, it keeps the compiler from sinking the
// loads past the barrier to their uses (which would wait for each of them in
// turn); the wait it implies covers the older loads only.
template <int M>
__device__ __forceinline__ void xf_lanes_hold(XfLanes<M> &l) {
#pragma unroll
  for (int k = 0; k < M; ++k)
    asm volatile("" : "+v"(l.x[k]), "+v"(l.p[k]), "+v"(l.c[k]), "+v"(l.s[k]), "+v"(l.scale[k]),
                 "+v"(l.zero[k]));
}

template <int IN, int M>
__device__ __forceinline__ void xf_lane_load_one(XfLanes<M> &l, int k, const RowXf &x, int t,
                                                 uint32_t h, bool rot, const char *row,
                                                 const float *cr, const float *sr, uint32_t e) {
  l.x[k] = xf_raw_t<IN>(row, e);
  if (x.out_bytes == 1) xf_params(x, t, h, e, l.scale[k], l.zero[k]);
  l.p[k] = 0;
  l.c[k] = l.s[k] = 0.0f;
  if (rot) {  // an unrotated element loads a pair it will not use
    bool first;
    uint32_t j, pe;
    xf_pair(x, min(e, uint32_t(2 * x.half) - 1), first, j, pe);
    l.p[k] = xf_raw_t<IN>(row, pe);
    l.c[k] = cr[j];
    l.s[k] = sr[j];
  }
}

template <int IN, int M>
__device__ __forceinline__ void xf_lanes_load_t(XfLanes<M> &l, const RowXf &x, int t, uint32_t h,
                                                bool rot, const char *row, const float *cr,
                                                const float *sr, uint32_t lane, uint32_t n,
                                                uint32_t D, uint32_t m) {
#pragma unroll
  for (int k = 0; k < M; ++k) {
    l.x[k] = l.p[k] = 0, l.c[k] = l.s[k] = 0.0f;
    l.scale[k] = 1.0f, l.zero[k] = 0;
  }
  if (M == 1 || m == 1) {  // the usual row: one element per lane, straight-line
    xf_lane_load_one<IN>(l, 0, x, t, h, rot, row, cr, sr, min(lane, D - 1));
    return;
  }
#pragma unroll
  for (int k = 0; k < M; ++k)
    if (uint32_t(k) < m)  // uniform
      xf_lane_load_one<IN>(l, k, x, t, h, rot, row, cr, sr, min(lane + k * n, D - 1));
}

// One element a lane (M = 1), for one input type: every load is issued
// whatever the lane's role, and the values are held in the same branch, so
// the load phase is straight-line and its only wait is the hold's, after
// every load in flight (the shift's among them) has been issued. A branch
// join between the loads and the hold would cost a wait of its own (a value
// narrower than its register is widened after the join), and such a wait
// drains the shift's loads too. A lane that does not rotate (a V row, an
// element past rotary_dim) loads its own element as partner and the first
// entries of its table row, and ignores them.
template <int IN>
__device__ __forceinline__ void xf_lane_load1_t(XfLanes<1> &l, const RowXf &x, int t, uint32_t h,
                                                const char *row, int64_t pos, uint32_t lane,
                                                uint32_t D) {
  const uint32_t e = min(lane, D - 1);
  l.x[0] = xf_raw_t<IN>(row, e);
  l.p[0] = 0;
  l.c[0] = l.s[0] = 0.0f;
  l.scale[0] = 1.0f, l.zero[0] = 0;
  if (x.out_bytes == 1) xf_params(x, t, h, e, l.scale[0], l.zero[0]);
  if (x.cos) {  // uniform: tables given (the position has a row, K and V alike)
    const bool r = t == 0 && e < uint32_t(2 * x.half);
    bool first;
    uint32_t j, pe;
    xf_pair(x, min(e, uint32_t(2 * x.half) - 1), first, j, pe);
    const int64_t at = pos * x.half + (r ? j : 0);
    l.p[0] = xf_raw_t<IN>(row, r ? pe : e);
    l.c[0] = x.cos[at];
    l.s[0] = x.sin[at];
  }
  xf_lanes_hold(l);
}

// (t may differ between the waves of a workgroup; picking a scalar parameter
// may then become a load, issued here with the others; per-channel
// parameters are loads of their own)
template <int M>
__device__ __forceinline__ void xf_lanes_load(XfLanes<M> &l, const RowXf &x, int t, uint32_t h,
                                              const char *row, int64_t pos, uint32_t lane,
                                              uint32_t n, uint32_t D) {
  if constexpr (M == 1) {
    if (x.in_type == SWRT_XF_F32)
      xf_lane_load1_t<SWRT_XF_F32>(l, x, t, h, row, pos, lane, D);
    else if (x.in_type == SWRT_XF_BF16)
      xf_lane_load1_t<SWRT_XF_BF16>(l, x, t, h, row, pos, lane, D);
    else
      xf_lane_load1_t<SWRT_XF_F16>(l, x, t, h, row, pos, lane, D);
    return;
  }
  const uint32_t m = (D + n - 1) / n;  // elements per lane (uniform)
  const bool rot = t == 0 && x.cos;
  const float *cr = rot ? x.cos + pos * x.half : nullptr;
  const float *sr = rot ? x.sin + pos * x.half : nullptr;
  if (x.in_type == SWRT_XF_F32)
    xf_lanes_load_t<SWRT_XF_F32>(l, x, t, h, rot, row, cr, sr, lane, n, D, m);
  else if (x.in_type == SWRT_XF_BF16)
    xf_lanes_load_t<SWRT_XF_BF16>(l, x, t, h, rot, row, cr, sr, lane, n, D, m);
  else
    xf_lanes_load_t<SWRT_XF_F16>(l, x, t, h, rot, row, cr, sr, lane, n, D, m);
}

// The cache bits of lane element k (element e of the row; out_bytes wide, in
// the low bits)
template <int IN, int M>
__device__ __forceinline__ uint32_t xf_lane_encode_one(const XfLanes<M> &l, int k, const RowXf &x,
                                                       bool rot, uint32_t e) {
  const float v = xf_rotate<IN>(x, rot, e, l.x[k], l.p[k], l.c[k], l.s[k]);
  if (x.out_bytes == 4) return v != v ? 0x7FC00000u : __float_as_uint(v);
  if (x.out_bytes == 2) return x.out_type == SWRT_XF_BF16 ? xf_bf16(v) : xf_f16(v);
  return xf_byte(x, l.scale[k], l.zero[k], v);
}

template <int IN, int M>
__device__ __forceinline__ void xf_lanes_encode_t(XfLanes<M> &l, const RowXf &x, int t,
                                                  uint32_t lane, uint32_t n, uint32_t D) {
  const uint32_t m = (D + n - 1) / n;
  const bool rot = t == 0 && x.cos;
  if (M == 1 || m == 1) {
    if (lane < D) l.x[0] = xf_lane_encode_one<IN>(l, 0, x, rot, lane);
    return;
  }
#pragma unroll
  for (int k = 0; k < M; ++k) {
    const uint32_t e = lane + k * n;
    if (uint32_t(k) < m && e < D) l.x[k] = xf_lane_encode_one<IN>(l, k, x, rot, e);
  }
}

// Turn the held elements into their cache bits, in place (l.x), once their
// loads have returned and before the stores of the step: nothing computed
// after a store then reuses its data registers (on this target the store
// counter is the load counter, and such a reuse would wait for the store to
// complete before the wave could go on and end).
template <int M>
__device__ __forceinline__ void xf_lanes_encode(XfLanes<M> &l, const RowXf &x, int t,
                                                uint32_t lane, uint32_t n, uint32_t D) {
  if (x.in_type == SWRT_XF_F32)
    xf_lanes_encode_t<SWRT_XF_F32>(l, x, t, lane, n, D);
  else if (x.in_type == SWRT_XF_BF16)
    xf_lanes_encode_t<SWRT_XF_BF16>(l, x, t, lane, n, D);
  else
    xf_lanes_encode_t<SWRT_XF_F16>(l, x, t, lane, n, D);
}

// Store the encoded elements of the row at dst.
template <int M>
__device__ __forceinline__ void xf_lanes_put(const XfLanes<M> &l, const RowXf &x, char *dst,
                                             uint32_t lane, uint32_t n, uint32_t D) {
  const uint32_t m = M == 1 ? 1 : (D + n - 1) / n;
#pragma unroll
  for (int k = 0; k < M; ++k) {
    const uint32_t e = lane + k * n;
    if (uint32_t(k) < m && e < D) {
      if (x.out_bytes == 4)
        __builtin_nontemporal_store(l.x[k], reinterpret_cast<uint32_t *>(dst) + e);
      else if (x.out_bytes == 2)
        __builtin_nontemporal_store(uint16_t(l.x[k]), reinterpret_cast<uint16_t *>(dst) + e);
      else
        __builtin_nontemporal_store(uint8_t(l.x[k]), reinterpret_cast<uint8_t *>(dst) + e);
    }
  }
}

}  // namespace swrt
