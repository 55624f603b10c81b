// att_device.hpp -- helpers of the attention kernels' matrix-core value
// products (windowed and paged decode attention).
#pragma once

#include "swrt_device.hpp"

namespace swrt {

// the bf16 halves (top 16 bits) of two binary32 values, a in the low half
__device__ __forceinline__ uint32_t bf16_pack_hi(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// four binary32 values as three bf16 parts each, packed in pairs: truncating
// to the top 8 significant bits leaves an exact remainder, so the three parts
// add up to the value exactly (24 significant bits). A bf16 matrix
// instruction with exact bf16 partners then takes the value at full binary32
// precision in three passes.
__device__ __forceinline__ void bf16_split3(const float (&x4)[4], uint32_t (&pb)[3][2]) {
  float part[3][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float x = x4[r];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      part[k][r] = __uint_as_float(__float_as_uint(x) & 0xFFFF0000u);
      x = x - part[k][r];  // exact
    }
    part[2][r] = x;  // the packing below keeps its top 16 bits: the truncation
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    pb[k][0] = bf16_pack_hi(part[k][0], part[k][1]);
    pb[k][1] = bf16_pack_hi(part[k][2], part[k][3]);
  }
}

}  // namespace swrt
