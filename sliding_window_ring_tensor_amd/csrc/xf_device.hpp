// xf_device.hpp -- the row transform of a fused append.
//
// On its way into the cache a new K or V row (f32, f16 or bf16 elements) is
// read as float; K turns by RoPE at its absolute position (onnxruntime pull
// request "GQA support sliding_window_cache", "Summary of Changes": the append
// uses the cache-relative offset, RoPE the absolute position, bounded by the
// tables' own length and not by the capacity); then every element is written
// in the cache's type: f32, f16 or bf16 rounded to nearest even, or an affine
// INT8 / UINT8 code with the tensor's scalar scale and zero point, rounded
// half to even and saturated (onnx-light how-to "Persistent input/output
// feedback", section "Optional heterogeneous paged KV").
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
  float scale[2];               // K, V (integer codes)
  int32_t zero[2];
  int32_t lo, hi;               // code range
};

// positions [p0, p0 + n) all have table rows (always, without rotation)
__device__ __forceinline__ bool xf_positions_ok(const RowXf &x, int64_t p0, int64_t n) {
  return !x.cos || (p0 >= 0 && p0 <= x.max_pos - n);
}

__device__ __forceinline__ float xf_in(const RowXf &x, const char *row, uint32_t e) {
  if (x.in_type == SWRT_XF_F32) return reinterpret_cast<const float *>(row)[e];
  const uint16_t h = reinterpret_cast<const uint16_t *>(row)[e];
  if (x.in_type == SWRT_XF_BF16) return __uint_as_float(uint32_t(h) << 16);
  return float(__builtin_bit_cast(_Float16, h));
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

__device__ __forceinline__ int32_t xf_code(const RowXf &x, int t, float y) {
  if (y != y) return x.zero[t];
  float q = __builtin_rintf(y / x.scale[t]) + float(x.zero[t]);
  q = fminf(fmaxf(q, float(x.lo)), float(x.hi));
  return int32_t(q);
}

// element e of the row after the rotation (K with tables) or as it is
template <bool ROT>
__device__ __forceinline__ float xf_element(const RowXf &x, const char *row, const float *cr,
                                            const float *sr, uint32_t e) {
#pragma clang fp contract(off)
  float v = xf_in(x, row, e);
  if (ROT && e < uint32_t(2 * x.half)) {
    const uint32_t h = uint32_t(x.half);
    const bool first = x.interleaved ? (e & 1u) == 0 : e < h;
    const uint32_t j = x.interleaved ? e >> 1 : (first ? e : e - h);
    const uint32_t pe = x.interleaved ? (e ^ 1u) : (first ? e + h : e - h);
    const float p = xf_in(x, row, pe);
    const float vc = v * cr[j], ps = p * sr[j];
    v = first ? vc - ps : vc + ps;
  }
  return v;
}

template <int VEC, int OB, bool ROT>
__device__ __forceinline__ typename Word<VEC>::T xf_word_of(const RowXf &x, int t, const char *row,
                                                            const float *cr, const float *sr,
                                                            uint32_t i) {
  using W = typename Word<VEC>::T;
  constexpr int N = VEC / OB;  // elements in the word
  uint8_t b[VEC] = {};
  if constexpr (N >= 1) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const float v = xf_element<ROT>(x, row, cr, sr, i * N + k);
      if constexpr (OB == 4) {
        const uint32_t u = v != v ? 0x7FC00000u : __float_as_uint(v);
        __builtin_memcpy(b + 4 * k, &u, 4);
      } else if constexpr (OB == 2) {
        const uint16_t h = x.out_type == SWRT_XF_BF16 ? xf_bf16(v) : xf_f16(v);
        __builtin_memcpy(b + 2 * k, &h, 2);
      } else {
        b[k] = uint8_t(xf_code(x, t, v));  // two's complement bits for INT8
      }
    }
  }
  W w;
  __builtin_memcpy(&w, b, VEC);
  return w;
}

// Word i (VEC bytes of out_type elements) of the transform of `row`, tensor t
// (0 = K, rotated when tables are given; 1 = V) at absolute position pos.
// The cache's element alignment makes VEC a multiple of out_bytes.
template <int VEC>
__device__ __forceinline__ typename Word<VEC>::T xf_word(const RowXf &x, int t, const char *row,
                                                         int64_t pos, uint32_t i) {
  if (t == 0 && x.cos) {
    const float *cr = x.cos + pos * x.half, *sr = x.sin + pos * x.half;
    if (x.out_bytes == 1) return xf_word_of<VEC, 1, true>(x, t, row, cr, sr, i);
    if (x.out_bytes == 2) return xf_word_of<VEC, 2, true>(x, t, row, cr, sr, i);
    return xf_word_of<VEC, 4, true>(x, t, row, cr, sr, i);
  }
  if (x.out_bytes == 1) return xf_word_of<VEC, 1, false>(x, t, row, nullptr, nullptr, i);
  if (x.out_bytes == 2) return xf_word_of<VEC, 2, false>(x, t, row, nullptr, nullptr, i);
  return xf_word_of<VEC, 4, false>(x, t, row, nullptr, nullptr, i);
}

}  // namespace swrt
