// Device helpers shared by the libpkv kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlock = 16;  // tokens per cache block
constexpr int kWave = 64;   // CDNA wavefront
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// matrix-core operations (operand layouts, lane = 16 * j + c):
//   16x16x32 bf16: A lane holds A[m = c][k = 8j .. 8j+7], B lane holds
//                  B[k = 8j .. 8j+7][n = c]; C lane holds C[m = 4j + r][n = c].
//   16x16x16 bf16: as above with k = 4j .. 4j+3.
//   16x16x4  f32 : A[m = c][k = j], B[k = j][n = c].
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mma_bf16_k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16_k16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                    __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
// 32x32 output tile, k = 16: A lane (row l%32) holds A[row][8*(l/32) + 0..7],
// B lane (col l%32) holds B[8*(l/32) + 0..7][col], C element v of lane l is
// C[8*(v/4) + 4*(l/32) + v%4][l%32].
__device__ __forceinline__ f32x16 mma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32_k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// scalar math
// ---------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// cap * tanh(x / cap), scaled by log2(e) for the base-2 softmax.
// tanh(y) = 1 - 2 / (e^{2y} + 1): saturates to +-1 when e^{2y} over/underflows.
__device__ __forceinline__ float softcap_log2(float x, float cap, float inv_cap) {
  const float e = fast_exp2(x * inv_cap * (2.0f * kLog2e));
  const float th = 1.0f - 2.0f * fast_rcp(e + 1.0f);
  return (cap * kLog2e) * th;
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// round-to-nearest-even bf16 pair by the hardware conversion
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// x combined with the value of lane l ^ 32 (one cross-half lane swap)
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x combined over lanes l, l ^ 16, l ^ 32, l ^ 48 (lane swaps, no LDS)
__device__ __forceinline__ float quad_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return half_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quad_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return half_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// ---------------------------------------------------------------------------
// wave reductions / scans
// ---------------------------------------------------------------------------
__device__ __forceinline__ long long wave_sum_i64(long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Inclusive prefix sum over the 64 lanes in six DPP steps (no LDS round
// trips): row-local Hillis-Steele shifts by 1, 2, 4, 8 within each row of 16
// lanes, then the last lane of row 0 (2) added to row 1 (3), and the last
// lane of row 1 to rows 2 and 3.  The sum must fit in 32 bits.
__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}
__device__ __forceinline__ long long wave_incl_scan_i64(long long v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const long long t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// ---------------------------------------------------------------------------
// sequence geometry: the visible token range [vis_lo, L) and the cache
// blocks it touches, first_blk .. first_blk + nb - 1.
// ---------------------------------------------------------------------------
struct SeqSpan {
  int L_raw;      // context length as given
  int L;          // context length, clamped to [0, max_len]
  int vis_lo;     // first visible token (window), 0 without a window
  int first_blk;  // logical block holding vis_lo
  int nb;         // number of logical blocks the visible range touches
};

// max_len: the largest length the caller promised (and the block table can hold)
__device__ __forceinline__ SeqSpan seq_span(int L_raw, int window, int max_len) {
  SeqSpan s;
  s.L_raw = L_raw;
  s.L = min(max(L_raw, 0), max_len);
  s.vis_lo = (window > 0) ? max(0, s.L - window) : 0;
  s.first_blk = s.vis_lo / kBlock;
  s.nb = (s.L > 0) ? (s.L - 1) / kBlock - s.first_blk + 1 : 0;
  return s;
}

// AttentionSink tokens kept beside a window: tokens [0, sink) stay visible,
// and the walk visits the ns blocks holding them that lie before the
// window's first block, then the window's blocks.  Walk index j is logical
// block j < ns ? j : first_blk + j - ns.
struct SinkPart {
  int sink;  // visible sink tokens (0 without a window)
  int ns;    // sink blocks walked before first_blk
  __device__ __forceinline__ int blk(const SeqSpan& s, int j) const {
    return j < ns ? j : j - ns + s.first_blk;
  }
  __device__ __forceinline__ bool visible(const SeqSpan& s, int t) const {
    return (t < s.L) & ((t >= s.vis_lo) | (t < sink));
  }
};

__device__ __forceinline__ SinkPart sink_part(const SeqSpan& s, int window, int sink) {
  SinkPart k;
  k.sink = (window > 0) ? min(max(sink, 0), s.L) : 0;
  k.ns = min((k.sink + kBlock - 1) / kBlock, s.first_blk);
  return k;
}

// the span of a sequence whose walk also covers its sink blocks
__device__ __forceinline__ SeqSpan seq_span_sink(int L_raw, int window, int max_len, int sink) {
  SeqSpan s = seq_span(L_raw, window, max_len);
  if (s.L > 0) s.nb += sink_part(s, window, sink).ns;
  return s;
}

}  // namespace pkv
