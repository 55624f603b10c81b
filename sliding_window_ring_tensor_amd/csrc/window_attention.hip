// window_attention.hip -- one-token decode attention over windowed caches on
// gfx950 (onnx-light-cpu "Persistent KV Cache and Decode Performance
// Roadmap", section "Phase 1: decode with contiguous KV cache": a streaming
// kernel that, per KV block, takes the query/K dot products, updates the
// online-softmax state and accumulates V without storing the score vector;
// query heads that share a KV head read each KV block once; scores, softmax
// and accumulation in fp32. The window is that of the pull request "GQA
// support sliding_window_cache": the query at position T - 1 sees the last W
// resident rows, [max(0, L - W), L).)
//
// One workgroup (4 waves) per (layer, b, kv head). Its G = Hq / Hkv query
// heads are held by every lane; a K or V row is split over LPR lanes of 8
// bytes each, so one wave covers 64 / LPR consecutive rows per step and the
// four waves interleave their steps (each load instruction of a wave reads
// 512 contiguous bytes). Each lane keeps an online-softmax state (m, l, o)
// per head for the rows it has seen; states merge exactly across the rows of
// a wave (lane shuffles) and across waves (LDS). Scores use exp2 with log2(e)
// folded into the scale.
#include "swrt_host.hpp"
#include "att_device.hpp"

namespace swrt {
namespace {

constexpr int kAttBlock = 256;  // 4 waves
constexpr int kAttWaves = kAttBlock / 64;
// steps (of 64 / LPR rows) a wave loads at once, a block of the stream;
// fewer for large groups, whose per-head state fills the registers
constexpr int att_steps(int G) { return G <= 4 ? 8 : G == 8 ? 4 : 2; }
// per-wave states published through LDS: G * LPR lanes' worth at most 256
constexpr bool att_supported(int LPR, int G) { return G * LPR <= 256; }

struct AttArgs {
  const char *q[kMaxLayers];
  const char *k[kMaxLayers];
  const char *v[kMaxLayers];
  char *out[kMaxLayers];
  const int32_t *L;
  uint32_t *flags;
  float scale_log2;  // scale * log2(e)
  int32_t W, B, Hq, Hkv, C, D, out_type;
  int32_t items;   // n_layers * B * Hkv (* chunks for the matrix-core kernel)
  int32_t chunks;  // matrix-core kernel: groups of up to 16 query heads per KV head
};

template <int ELEM>
__device__ __forceinline__ float att_decode(uint32_t r) {
  if constexpr (ELEM == SWRT_XF_F32)
    return __uint_as_float(r);
  else if constexpr (ELEM == SWRT_XF_BF16)
    return __uint_as_float(r << 16);
  else
    return float(__builtin_bit_cast(_Float16, uint16_t(r)));
}

// the EPL elements of an 8-byte chunk
template <int ELEM, int EPL>
__device__ __forceinline__ void att_unpack(u32x2 w, float (&x)[EPL]) {
  if constexpr (ELEM == SWRT_XF_F32) {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
  } else {
    x[0] = att_decode<ELEM>(w.x & 0xFFFFu);
    x[1] = att_decode<ELEM>(w.x >> 16);
    x[2] = att_decode<ELEM>(w.y & 0xFFFFu);
    x[3] = att_decode<ELEM>(w.y >> 16);
  }
}

// sums over aligned groups of N lanes (N a power of two, 1 .. 64) of K values
// at once, level by level, so the lane exchanges of different values
// interleave; every lane of a group gets the group's sums
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF,
                                                        false));
}

template <int N, int K>
__device__ __forceinline__ void group_sums(float (&x)[K]) {
#pragma unroll
  for (int k = 0; k < K; ++k)
    if constexpr (N >= 2) x[k] = dpp_add<0xB1>(x[k]);  // lanes i ^ 1
#pragma unroll
  for (int k = 0; k < K; ++k)
    if constexpr (N >= 4) x[k] = dpp_add<0x4E>(x[k]);  // lanes i ^ 2
#pragma unroll
  for (int k = 0; k < K; ++k)
    if constexpr (N >= 8) x[k] = dpp_add<0x141>(x[k]);  // the other quad of the half row
#pragma unroll
  for (int k = 0; k < K; ++k)
    if constexpr (N >= 16) x[k] = dpp_add<0x140>(x[k]);  // the other half of the row
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if constexpr (N >= 32) x[k] += __shfl_xor(x[k], 16);
    if constexpr (N >= 64) x[k] += __shfl_xor(x[k], 32);
  }
}

// A block of S scores (masked rows: -inf) joins a head's online-softmax
// state: the new maximum, the factor f that rescales the old state and the
// weights p of the rows. Each score is rounded once and compared with
// itself: a fused multiply-add of dot * scale - max would leave that
// rounding as a residual and give the row at the maximum a weight other
// than 1. Selects, not branches, handle a state that has seen nothing.
template <int S>
__device__ __forceinline__ void att_block(const float (&dot)[S], const bool (&ok)[S],
                                          float scale_log2, float &m, float &f, float (&p)[S]) {
#pragma clang fp contract(off)
  float sc[S];
  float mn = m;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    sc[s] = ok[s] ? dot[s] * scale_log2 : -INFINITY;
    mn = fmaxf(mn, sc[s]);
  }
  const bool none = mn == -INFINITY;  // nothing seen yet
  f = none ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
  for (int s = 0; s < S; ++s) p[s] = none ? 0.0f : __builtin_amdgcn_exp2f(sc[s] - mn);
  m = mn;
}

// merge online-softmax state b into a (same rows never counted twice)
template <int EPL>
__device__ __forceinline__ void att_merge(float &m, float &l, float (&o)[EPL], float mb, float lb,
                                          const float (&ob)[EPL]) {
  const float mn = fmaxf(m, mb);
  if (mn == -INFINITY) return;  // both empty
  const float fa = __builtin_amdgcn_exp2f(m - mn), fb = __builtin_amdgcn_exp2f(mb - mn);
  l = l * fa + lb * fb;
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = o[e] * fa + ob[e] * fb;
  m = mn;
}

template <int ELEM, int LPR, int G>
__global__ __launch_bounds__(kAttBlock) void window_attention_kernel(AttArgs a) {
  constexpr int EPL = ELEM == SWRT_XF_F32 ? 2 : 4;  // elements per 8-byte chunk
  constexpr int RW = 64 / LPR;                      // rows per wave step
  constexpr int kAttStep = att_steps(G);
  const uint32_t bid = blockIdx.x;
  const uint32_t g = bid % uint32_t(a.Hkv), b = (bid / uint32_t(a.Hkv)) % uint32_t(a.B);
  const uint32_t layer = bid / uint32_t(a.Hkv * a.B);
  const int64_t L = a.L[b];
  if (L < 0 || L > a.C) {  // no partial output for this entry
    if (a.flags && g == 0 && layer == 0 && threadIdx.x == 0) atomicOr(a.flags, SWRT_FLAG_BAD_LENGTHS);
    return;
  }
  const int64_t r0 = L > a.W ? L - a.W : 0;
  const uint32_t lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const uint32_t c = lane % LPR, rr = lane / LPR;  // chunk of the row, row of the step
  const uint32_t es = ELEM == SWRT_XF_F32 ? 4 : 2;
  const uint64_t row_bytes = uint64_t(a.D) * es;
  const uint64_t kv_off = (uint64_t(b) * a.Hkv + g) * uint64_t(a.C) * row_bytes;
  const char *kb = a.k[layer] + kv_off + c * 8;
  const char *vb = a.v[layer] + kv_off + c * 8;

  // this lane's chunk of every query head of the group
  float q[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const u32x2 w = *reinterpret_cast<const u32x2 *>(
        a.q[layer] + ((uint64_t(b) * a.Hq + g * G + j) * row_bytes) + c * 8);
    att_unpack<ELEM, EPL>(w, q[j]);
  }

  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[j][e] = 0.0f;
  }

  // rows of this wave: r0 + (s * waves + wave) * RW + rr, s = 0, 1, ...
  const int64_t stride = int64_t(kAttWaves) * RW;
  for (int64_t base = r0 + int64_t(wave) * RW; base < L; base += kAttStep * stride) {
    // every load of the block first (steps past the window, uniform in the
    // wave, load nothing), then the rows one step at a time
    u32x2 kw[kAttStep], vw[kAttStep];
#pragma unroll
    for (int s = 0; s < kAttStep; ++s) {
      if (base + s * stride < L) {
        const int64_t r = base + s * stride + rr;
        const int64_t rc = r < L ? r : L - 1;  // lanes past the window repeat a valid row
        kw[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(kb + rc * row_bytes));
        vw[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(vb + rc * row_bytes));
      } else {  // zeros: a masked row's weight 0 times its V must stay 0
        kw[s] = u32x2{0u, 0u};
        vw[s] = u32x2{0u, 0u};
      }
    }
    // scores of the block: per step, every head's partial dot, then their
    // lane sums together (rows past the window compute on a repeated row
    // and are masked)
    bool ok[kAttStep];
    float dots[G][kAttStep];
#pragma unroll
    for (int s = 0; s < kAttStep; ++s) {
      ok[s] = base + s * stride + rr < L;
      float kx[EPL];
      att_unpack<ELEM, EPL>(kw[s], kx);
      float d[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        d[j] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d[j] += q[j][e] * kx[e];
      }
      group_sums<LPR, G>(d);
#pragma unroll
      for (int j = 0; j < G; ++j) dots[j][s] = d[j];
    }
    // one rescale per head, then the block's weighted rows
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float f, p[kAttStep];
      att_block<kAttStep>(dots[j], ok, a.scale_log2, m[j], f, p);
      l[j] *= f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[j][e] *= f;
#pragma unroll
      for (int s = 0; s < kAttStep; ++s) {
        float vx[EPL];
        att_unpack<ELEM, EPL>(vw[s], vx);
        l[j] += p[s];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] += p[s] * vx[e];
      }
    }
  }

  // merge the RW row groups of the wave (lanes c, c + LPR, c + 2 LPR, ...)
#pragma unroll
  for (int off = LPR; off < 64; off *= 2) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float ob[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) ob[e] = __shfl_xor(o[j][e], off);
      att_merge<EPL>(m[j], l[j], o[j], __shfl_xor(m[j], off), __shfl_xor(l[j], off), ob);
    }
  }
  // then the waves, through LDS: lanes rr == 0 of each wave publish
  __shared__ float st[kAttWaves][G][LPR][EPL + 2];
  if (rr == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      st[wave][j][c][0] = m[j];
      st[wave][j][c][1] = l[j];
#pragma unroll
      for (int e = 0; e < EPL; ++e) st[wave][j][c][2 + e] = o[j][e];
    }
  }
  __syncthreads();
  if (wave != 0 || rr != 0) return;
#pragma unroll
  for (int w = 1; w < kAttWaves; ++w) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float ob[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) ob[e] = st[w][j][c][2 + e];
      att_merge<EPL>(m[j], l[j], o[j], st[w][j][c][0], st[w][j][c][1], ob);
    }
  }
  // normalise and write head g * G + j's chunk c
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float inv = l[j] > 0.0f ? 1.0f / l[j] : 0.0f;  // an empty window gives zeros
    char *dst = a.out[layer] + (uint64_t(b) * a.Hq + g * G + j) * uint64_t(a.D) *
                                   (a.out_type == SWRT_XF_F32 ? 4 : 2);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float y = o[j][e] * inv;
      const uint32_t idx = c * EPL + e;
      if (a.out_type == SWRT_XF_F32)
        reinterpret_cast<float *>(dst)[idx] = y;
      else if (a.out_type == SWRT_XF_BF16)
        reinterpret_cast<uint16_t *>(dst)[idx] = xf_bf16(y);
      else
        reinterpret_cast<uint16_t *>(dst)[idx] = xf_f16(y);
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core path (16-bit caches). Both contractions of a KV head's window
// run on MFMA, so the VALU keeps only the softmax of each (row, head) score
// once, instead of per lane of a row as above.
//   scores  S^T = K Q^T with v_mfma_f32_16x16x32_{bf16,f16}: 16 window rows
//           (M) by 16 head slots (N; heads >= G are zero), head_dim reduced
//           32 per instruction. Products of two 16-bit values are exact in
//           fp32; the sum of head_dim of them is rounded in fp32.
//   values  O^T = V^T P^T with v_mfma_f32_16x16x4_f32: 16 output dimensions
//           by 16 head slots, 4 rows per instruction, the weights P in fp32
//           (not rounded to 16 bits), V widened exactly to fp32.
// Lane l holds head slot j = l % 16 of every accumulator and rows
// q + 4 r (q = l / 16, r = 0..3) of each 16-row tile of scores; the key
// operand carries tile row pk(i) = i / 4 + 4 (i % 4) at matrix row i, so the
// scores' row 4 q + r is tile row q + 4 r and the value product's k-th
// instruction (rows 4 k .. 4 k + 3 of the tile, one per lane group q) takes
// its weights straight from each lane's r = k score. Dimension
// MT * i + m (MT = head_dim / 16) sits at matrix row i of output tile m, so a
// lane reads MT consecutive elements of a V row and ends holding 4 MT
// consecutive output dimensions, 4 MT q .. 4 MT q + 4 MT - 1, of its head.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short att_s16x4 __attribute__((ext_vector_type(4)));

template <int ELEM>
__device__ __forceinline__ f32x4 score_mfma(u32x4 k, u32x4 q, f32x4 acc) {
  if constexpr (ELEM == SWRT_XF_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                   __builtin_bit_cast(bf16x8, q), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                  __builtin_bit_cast(f16x8, q), acc, 0, 0, 0);
}

// NB bytes (4, 8, 16 or 32) of a row as 32-bit words, streamed
template <int NB>
__device__ __forceinline__ void att_load_words(const char *p, uint32_t (&w)[NB / 4]) {
  if constexpr (NB == 4) {
    w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
  } else if constexpr (NB == 8) {
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    w[0] = x.x;
    w[1] = x.y;
  } else if constexpr (NB == 12) {  // head_dim 96: 4-byte aligned chunks
#pragma unroll
    for (int i = 0; i < 3; ++i) w[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p) + i);
  } else if constexpr (NB == 24) {  // head_dim 192: 8-byte aligned chunks
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p) + i);
      w[2 * i] = x.x;
      w[2 * i + 1] = x.y;
    }
  } else {
    static_assert(NB % 16 == 0, "V chunk bytes");
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p) + i);
      w[4 * i] = x.x;
      w[4 * i + 1] = x.y;
      w[4 * i + 2] = x.z;
      w[4 * i + 3] = x.w;
    }
  }
}

// element e of a lane's packed 16-bit V elements, widened exactly
template <int ELEM, int NW32>
__device__ __forceinline__ float att_elem(const uint32_t (&w)[NW32], int e) {
  const uint32_t x = w[e / 2];
  if constexpr (ELEM == SWRT_XF_BF16)
    return __uint_as_float(e % 2 ? x & 0xFFFF0000u : x << 16);
  else
    return float(__builtin_bit_cast(_Float16, uint16_t(e % 2 ? x >> 16 : x & 0xFFFFu)));
}

// merge state b into a, branch-free (an empty state has m = -inf, l = 0, o = 0)
template <int N>
__device__ __forceinline__ void att_merge_flat(float &m, float &l, f32x4 (&o)[N], float mb,
                                               float lb, const f32x4 (&ob)[N]) {
  const float mn = fmaxf(m, mb);
  const bool none = mn == -INFINITY;
  const float fa = none ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
  const float fb = none ? 0.0f : __builtin_amdgcn_exp2f(mb - mn);
  l = l * fa + lb * fb;
#pragma unroll
  for (int i = 0; i < N; ++i) o[i] = o[i] * fa + ob[i] * fb;
  m = mn;
}

constexpr int att_tiles(int D) { return D <= 32 ? 4 : D == 64 ? 2 : 1; }
constexpr bool kAttPrefetch = false;

// One (layer, b, kv head) per NW waves: NW = 1 puts four of them in a
// workgroup, NW = 4 splits one window's 16-row tiles over the four waves and
// merges their states through LDS.
template <int ELEM, int D, int NW>
__global__ __launch_bounds__(kAttBlock) void window_attention_mfma(AttArgs a) {
  constexpr int KS = D / 32;  // score instructions per tile
  constexpr int MT = D / 16;  // output tiles
  constexpr int VB = D / 8;   // bytes of a V row per lane (MT elements)
  constexpr int T = att_tiles(D);  // tiles per block of the stream
  constexpr uint32_t row_bytes = D * 2;
  const uint32_t lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const uint32_t j = lane % 16, qg = lane / 16;
  const uint32_t item = blockIdx.x * (kAttWaves / NW) + wave / NW, ws = wave % NW;
  if (item >= uint32_t(a.items)) return;  // NW = 4: the whole workgroup
  // an item is (layer, b, kv head, chunk): the chunk's query heads are
  // 16 chunk .. 16 chunk + 15 of the group (a group of more than 16 heads is
  // split over consecutive items, whose waves read the same K/V rows)
  const uint32_t chunk = item % uint32_t(a.chunks), win = item / uint32_t(a.chunks);
  const uint32_t g = win % uint32_t(a.Hkv), b = (win / uint32_t(a.Hkv)) % uint32_t(a.B);
  const uint32_t layer = win / uint32_t(a.Hkv * a.B);
  const int64_t L = a.L[b];
  if (L < 0 || L > a.C) {  // no partial output for this entry (uniform in the workgroup for NW = 4)
    if (a.flags && g == 0 && chunk == 0 && layer == 0 && ws == 0 && lane == 0)
      atomicOr(a.flags, SWRT_FLAG_BAD_LENGTHS);
    return;
  }
  // row numbers stay below capacity + 16 < 2^31 (checked on the host)
  const int32_t Li = int32_t(L), r0 = Li > a.W ? Li - a.W : 0, last = Li - 1;
  const int G = a.Hq / a.Hkv;
  const int hs = int(16 * chunk + j);  // this lane's head within the group
  const bool head = hs < G;
  const uint64_t kv_off = (uint64_t(b) * a.Hkv + g) * uint64_t(a.C) * row_bytes;
  const char *kb = a.k[layer] + kv_off + 16 * qg;
  const char *vb = a.v[layer] + kv_off + VB * j;

  // query operand: head slot j's 8 elements of each 32-element step (zeros
  // for slots past the group; they read head 0's row to stay in bounds)
  u32x4 qo[KS];
  {
    const char *qp = a.q[layer] + (uint64_t(b) * a.Hq + g * G + (head ? hs : 0)) * row_bytes +
                     16 * qg;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 x = *reinterpret_cast<const u32x4 *>(qp + 64 * s);
      qo[s] = head ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float m = -INFINITY, l = 0.0f;
  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int32_t n_tiles = (Li - r0 + 15) / 16;
  const int32_t pk = (j >> 2) + 4 * (j & 3);  // tile row of this lane's key operand
  // Blocks of T tiles. A block wholly inside the window loads from two
  // pointers with constant offsets and needs no mask; the last one clamps
  // rows past L to row L - 1 (masked), and tiles past the window (uniform in
  // the wave) load nothing.
  struct Tiles {
    u32x4 kw[T][KS];
    uint32_t vw[T][4][VB / 4];
  };
  auto load = [&](Tiles &d, int32_t t0) {
    if (r0 + 16 * (t0 + T) <= Li) {
      const char *kr = kb + uint64_t(uint32_t(r0 + 16 * t0 + pk)) * row_bytes;
      const char *vr = vb + uint64_t(uint32_t(r0 + 16 * t0 + int32_t(qg))) * row_bytes;
#pragma unroll
      for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
          d.kw[t][s] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4 *>(kr + 16 * t * row_bytes + 64 * s));
#pragma unroll
        for (int c = 0; c < 4; ++c) att_load_words<VB>(vr + (16 * t + 4 * c) * row_bytes, d.vw[t][c]);
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (t0 + t < n_tiles) {
        const int32_t tb = r0 + 16 * (t0 + t);
        const char *kr = kb + uint64_t(uint32_t(min(tb + pk, last))) * row_bytes;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          d.kw[t][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kr + 64 * s));
#pragma unroll
        for (int c = 0; c < 4; ++c)
          att_load_words<VB>(
              vb + uint64_t(uint32_t(min(tb + 4 * c + int32_t(qg), last))) * row_bytes,
              d.vw[t][c]);
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) d.kw[t][s] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i = 0; i < VB / 4; ++i) d.vw[t][c][i] = 0u;
      }
    }
  };
  Tiles cur;
  if constexpr (kAttPrefetch) load(cur, int32_t(ws) * T);
  for (int32_t t0 = int32_t(ws) * T; t0 < n_tiles; t0 += NW * T) {
    // with prefetch, the next block's loads are issued before this block's
    // arithmetic, so a wave keeps two blocks of reads in flight
    Tiles nxt;
    if constexpr (kAttPrefetch)
      load(nxt, t0 + NW * T);
    else
      load(cur, t0);
    const auto &kw = cur.kw;
    const auto &vw = cur.vw;
    // scores, then the block's softmax update: one maximum per head over the
    // wave (the value product sums every lane group's rows), weights in
    // fp32. Masked after the scale, so a negative scale cannot flip a -inf.
    float x[T][4];
    float bm = -INFINITY;
    {
#pragma clang fp contract(off)
      f32x4 sc[T];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        sc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KS; ++s) sc[t] = score_mfma<ELEM>(kw[t][s], qo[s], sc[t]);
      }
      if (r0 + 16 * (t0 + T) <= Li) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[t][r] = sc[t][r] * a.scale_log2;
            bm = fmaxf(bm, x[t][r]);
          }
      } else {
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const int32_t tb = r0 + 16 * (t0 + t) + int32_t(qg);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[t][r] = tb + 4 * r < Li ? sc[t][r] * a.scale_log2 : -INFINITY;
            bm = fmaxf(bm, x[t][r]);
          }
        }
      }
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    // The reference maximum m moves only when the block's exceeds it by more
    // than 2^8 (log2 units): weights exp2(x - m) stay below 2^8, which costs
    // no precision in fp32, and most blocks skip the rescale of the state.
    // A single visible row still gets weight exp2(0) = 1 exactly.
    float p[T][4];
    {
#pragma clang fp contract(off)
      const bool move = bm > m + 8.0f;  // m = -inf: the first block with a visible row
      const float mn = move ? bm : m;
      if (__builtin_amdgcn_ballot_w64(move && m != -INFINITY)) {
        const float f = move ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;
        l *= f;
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i] *= f;
      }
      const bool none = mn == -INFINITY;  // nothing seen yet
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[t][r] = none ? 0.0f : __builtin_amdgcn_exp2f(x[t][r] - mn);
          l += p[t][r];
        }
      m = mn;
    }
    // the block's weighted rows. bf16 V: v_mfma_f32_16x16x16_bf16, whose four
    // k-slots per lane are the four rows 4 c + q a lane holds (and whose
    // weights it holds too), each binary32 weight as three exact bf16 parts;
    // f16 V: v_mfma_f32_16x16x4_f32, one row per instruction
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if constexpr (ELEM == SWRT_XF_BF16) {
        uint32_t pb[3][2];
        bf16_split3(p[t], pb);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const uint32_t sel = i % 2 ? 0x07060302u : 0x05040100u;
          const u32x2 va{__builtin_amdgcn_perm(vw[t][1][i / 2], vw[t][0][i / 2], sel),
                         __builtin_amdgcn_perm(vw[t][3][i / 2], vw[t][2][i / 2], sel)};
#pragma unroll
          for (int k = 2; k >= 0; --k)  // the small parts first
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(att_s16x4, va),
                __builtin_bit_cast(att_s16x4, u32x2{pb[k][0], pb[k][1]}), acc[i], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i = 0; i < MT; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(att_elem<ELEM, VB / 4>(vw[t][c], i),
                                                          p[t][c], acc[i], 0, 0, 0);
      }
    }
    if constexpr (kAttPrefetch) cur = nxt;
  }

  if constexpr (NW > 1) {  // the waves' states, merged by wave 0 through LDS
    __shared__ float st[NW - 1][2 + 4 * MT][64];
    if (ws > 0) {
      st[ws - 1][0][lane] = m;
      st[ws - 1][1][lane] = l;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[ws - 1][2 + 4 * i + r][lane] = acc[i][r];
    }
    __syncthreads();
    if (ws > 0) return;
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) {
      f32x4 ob[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) ob[i][r] = st[w][2 + 4 * i + r][lane];
      att_merge_flat<MT>(m, l, acc, st[w][0][lane], st[w][1][lane], ob);
    }
  }
  // the head's weight sum over the four lane groups
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (!head) return;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;  // an empty window gives zeros
  // dimensions 4 MT qg + e, e = MT r + i, of head g * G + j
  float y[4 * MT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < MT; ++i) y[MT * r + i] = acc[i][r] * inv;
  const uint64_t orow = uint64_t(b) * a.Hq + g * G + hs;
  if (a.out_type == SWRT_XF_F32) {
    u32x4 *dst = reinterpret_cast<u32x4 *>(a.out[layer] + (orow * D + 4 * MT * qg) * 4);
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
    u32x4 *dst = reinterpret_cast<u32x4 *>(a.out[layer] + (orow * D + 4 * MT * qg) * 2);
#pragma unroll
    for (int c = 0; c < MT / 2; ++c) dst[c] = u32x4{h[4 * c], h[4 * c + 1], h[4 * c + 2], h[4 * c + 3]};
  }
}

template <int ELEM, int D>
int launch_mfma(const AttArgs &a, int nw, hipStream_t s) {
  if (nw == 1) {
    const uint32_t grid = (uint32_t(a.items) + kAttWaves - 1) / kAttWaves;
    hipLaunchKernelGGL((window_attention_mfma<ELEM, D, 1>), dim3(grid), dim3(kAttBlock), 0, s, a);
  } else {
    hipLaunchKernelGGL((window_attention_mfma<ELEM, D, kAttWaves>), dim3(uint32_t(a.items)),
                       dim3(kAttBlock), 0, s, a);
  }
  return launch_status();
}

template <int ELEM>
int launch_mfma_d(const AttArgs &a, int nw, hipStream_t s) {
  switch (a.D) {
    case 32: return launch_mfma<ELEM, 32>(a, nw, s);
    case 64: return launch_mfma<ELEM, 64>(a, nw, s);
    case 96: return launch_mfma<ELEM, 96>(a, nw, s);
    case 128: return launch_mfma<ELEM, 128>(a, nw, s);
    case 192: return launch_mfma<ELEM, 192>(a, nw, s);
    default: return launch_mfma<ELEM, 256>(a, nw, s);
  }
}

template <int ELEM, int LPR, int G>
int launch_one(const AttArgs &a, uint32_t grid, hipStream_t s) {
  if constexpr (att_supported(LPR, G)) {
    hipLaunchKernelGGL((window_attention_kernel<ELEM, LPR, G>), dim3(grid), dim3(kAttBlock), 0, s,
                       a);
    return launch_status();
  } else {
    return SWRT_E_UNSUPPORTED;  // refused on the host before this point
  }
}

template <int ELEM, int LPR>
int launch_g(const AttArgs &a, int G, uint32_t grid, hipStream_t s) {
  switch (G) {
    case 1: return launch_one<ELEM, LPR, 1>(a, grid, s);
    case 2: return launch_one<ELEM, LPR, 2>(a, grid, s);
    case 4: return launch_one<ELEM, LPR, 4>(a, grid, s);
    case 8: return launch_one<ELEM, LPR, 8>(a, grid, s);
    default: return launch_one<ELEM, LPR, 16>(a, grid, s);
  }
}

template <int ELEM>
int launch_lpr(const AttArgs &a, int lpr, int G, uint32_t grid, hipStream_t s) {
  switch (lpr) {
    case 8: return launch_g<ELEM, 8>(a, G, grid, s);
    case 16: return launch_g<ELEM, 16>(a, G, grid, s);
    case 32: return launch_g<ELEM, 32>(a, G, grid, s);
    default: return launch_g<ELEM, 64>(a, G, grid, s);
  }
}

}  // namespace
}  // namespace swrt

using namespace swrt;

extern "C" int swrt_window_attention(int n_layers, const void *const *q,
                                     const void *const *k_caches, const void *const *v_caches,
                                     void *const *out, const int32_t *cache_total_lens,
                                     int window, int batch, int q_heads, int kv_heads,
                                     int capacity, int head_dim, float scale, int elem_type,
                                     int out_type, uint32_t *d_flags, void *stream) {
  if (n_layers < 0 || n_layers > kMaxLayers || batch < 0 || q_heads < 0 || kv_heads < 1 ||
      capacity < 1 || head_dim < 0 || window < 1)
    return SWRT_E_INVALID_ARG;
  if (elem_type != SWRT_XF_F32 && elem_type != SWRT_XF_F16 && elem_type != SWRT_XF_BF16)
    return SWRT_E_INVALID_ARG;
  if (out_type != SWRT_XF_F32 && out_type != SWRT_XF_F16 && out_type != SWRT_XF_BF16)
    return SWRT_E_INVALID_ARG;
  if (q_heads % kv_heads) return SWRT_E_INVALID_ARG;
  if (capacity > INT32_MAX - 32) return SWRT_E_UNSUPPORTED;  // row numbers in int32
  if (!(scale == scale) || scale > 3.4028235e38f || scale < -3.4028235e38f) return SWRT_E_INVALID_ARG;
  if (n_layers == 0 || batch == 0 || q_heads == 0 || head_dim == 0) return SWRT_OK;
  const int G = q_heads / kv_heads;
  // the VALU kernel is built for these group sizes; the matrix-core one takes any
  const bool valu_group = G == 1 || G == 2 || G == 4 || G == 8 || G == 16;
  const int64_t es = elem_type == SWRT_XF_F32 ? 4 : 2, oes = out_type == SWRT_XF_F32 ? 4 : 2;
  const int64_t row = int64_t(head_dim) * es;
  const int64_t lpr = row / 8;
  // the VALU kernel's rows: 8, 16, 32 or 64 lanes of 8 bytes; the matrix-core
  // kernel's head dims: multiples of 32 up to 256 that it is built for
  const bool valu_shape = row % 8 == 0 && (lpr == 8 || lpr == 16 || lpr == 32 || lpr == 64);
  const bool mfma_shape = elem_type != SWRT_XF_F32 &&
                          (head_dim == 32 || head_dim == 64 || head_dim == 96 || head_dim == 128 ||
                           head_dim == 192 || head_dim == 256);
  if (!valu_shape && !mfma_shape) return SWRT_E_UNSUPPORTED;
  // 16-bit caches take the matrix-core kernel, 16-byte aligned operands
  // needed; fp32 caches (or 8-byte aligned operands) the VALU one
  bool mfma = mfma_shape;
  if (!mfma && (!valu_group || G * lpr > 256)) return SWRT_E_UNSUPPORTED;  // see att_supported
  if (!q || !k_caches || !v_caches || !out || !cache_total_lens) return SWRT_E_INVALID_ARG;
  // batch, heads, capacity, head_dim < 2^31: their pairwise products fit
  int64_t bkc, bqd, cache_bytes, q_bytes, o_bytes, items;
  if (!mul_ok(int64_t(batch) * kv_heads, capacity, &bkc) || !mul_ok(bkc, row, &cache_bytes) ||
      !mul_ok(int64_t(batch) * q_heads, row, &q_bytes) ||
      !mul_ok(int64_t(batch) * q_heads, head_dim, &bqd) || !mul_ok(bqd, oes, &o_bytes))
    return SWRT_E_UNSUPPORTED;
  const int chunks = int((int64_t(G) + 15) / 16);  // the matrix-core kernel's items per window
  if (!mul_ok(int64_t(n_layers) * batch, int64_t(kv_heads) * chunks, &items) ||
      items >= (int64_t(1) << 31))
    return SWRT_E_UNSUPPORTED;
  Range ranges[4 * kMaxLayers + 2];
  int nr = 0;
  AttArgs a;
  for (int l = 0; l < n_layers; ++l) {
    if (!q[l] || !k_caches[l] || !v_caches[l] || !out[l]) return SWRT_E_INVALID_ARG;
    if (addr_of(q[l]) % 8 || addr_of(k_caches[l]) % 8 || addr_of(v_caches[l]) % 8 ||
        addr_of(out[l]) % uint64_t(oes))
      return SWRT_E_INVALID_ARG;
    if (addr_of(q[l]) % 16 || addr_of(k_caches[l]) % 16 || addr_of(v_caches[l]) % 16 ||
        addr_of(out[l]) % 16)
      mfma = false;
    ranges[nr++] = range(q[l], uint64_t(q_bytes), false);
    ranges[nr++] = range(k_caches[l], uint64_t(cache_bytes), false);
    ranges[nr++] = range(v_caches[l], uint64_t(cache_bytes), false);
    ranges[nr++] = range(out[l], uint64_t(o_bytes), true);
    a.q[l] = static_cast<const char *>(q[l]);
    a.k[l] = static_cast<const char *>(k_caches[l]);
    a.v[l] = static_cast<const char *>(v_caches[l]);
    a.out[l] = static_cast<char *>(out[l]);
  }
  if (addr_of(cache_total_lens) % 4 || addr_of(d_flags) % 4) return SWRT_E_INVALID_ARG;
  ranges[nr++] = range(cache_total_lens, uint64_t(batch) * 4, false);
  ranges[nr++] = range(d_flags, 4, true);
  if (written_overlap(ranges, nr)) return SWRT_E_INVALID_ARG;
  a.L = cache_total_lens;
  a.flags = d_flags;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.W = window;
  a.B = batch;
  a.Hq = q_heads;
  a.Hkv = kv_heads;
  a.C = capacity;
  a.D = head_dim;
  a.out_type = out_type;
  static_assert(sizeof(AttArgs) <= 4096, "kernel arguments exceed 4 KiB");
  const uint32_t grid = uint32_t(n_layers) * uint32_t(batch) * uint32_t(kv_heads);
  a.items = int32_t(grid);
  a.chunks = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mfma) {
    // one wave per (layer, b, kv head, chunk of 16 query heads) once there
    // are enough of them to fill the chip, else four waves share each
    a.chunks = chunks;
    a.items = int32_t(grid * uint32_t(chunks));
    const int nw = uint32_t(a.items) >= 2048 ? 1 : kAttWaves;
    return elem_type == SWRT_XF_BF16 ? launch_mfma_d<SWRT_XF_BF16>(a, nw, s)
                                     : launch_mfma_d<SWRT_XF_F16>(a, nw, s);
  }
  if (!valu_shape || !valu_group || G * lpr > 256) return SWRT_E_UNSUPPORTED;  // misaligned 16-bit operands
  switch (elem_type) {
    case SWRT_XF_F32: return launch_lpr<SWRT_XF_F32>(a, int(lpr), G, grid, s);
    case SWRT_XF_F16: return launch_lpr<SWRT_XF_F16>(a, int(lpr), G, grid, s);
    default: return launch_lpr<SWRT_XF_BF16>(a, int(lpr), G, grid, s);
  }
}
