// Per-lane operand fragments for one 16-token cache block, and the two
// matrix-core steps of attention over it.
//
// Layout choice.  The pools use the vLLM/PagedAttention layout (GitHub
// README of "Inference Server", section "What's inside"):
//     K block (one kv head): [D/X][16][X]   (X = elements per 16 bytes)
//     V block (one kv head): [D][16]
// so that both matrix-core operands load straight from HBM, coalesced:
//
//  * S^T = K Q^T on 16x16x32 bf16 tiles, A = K (row m = token), B = Q^T
//    (column n = query row).  Lane 16j+c of step i needs token c, dims
//    8(4i+j) .. +8, which is the 16 bytes at (64 i + lane) * 16 in the K
//    block: every step is one fully linear 1 KiB wave load.
//  * The result C[m = 4j + r][n = c] leaves lane 16j+c holding the scores of
//    tokens 4j .. 4j+3 for query row c.  That is exactly the A operand of a
//    16x16x16 bf16 product P V (A[m = c][k = 4j .. 4j+3]), so P never leaves
//    registers.
//  * The V operand of that product, V[k = 4j .. 4j+3][n = c] for dims
//    16t .. 16t+15, is 8 contiguous bytes of the V block per lane; a wave
//    load covers 512 contiguous bytes.
//
// fp32 pools use 16x16x4 f32 products with the same row/column roles; a lane
// loads 16 bytes and feeds four consecutive k-steps from them.
#pragma once

#include "common.hpp"

namespace pkv {

// Workgroup shape of the attention kernels: four waves of 64 lanes.
constexpr int kThreads = 256;
constexpr int kWaves = 4;

// Wait states between a matrix-core result and its first reader.  The
// compiler's hazard padding does not always reach a read that follows the
// last matrix op across a branch (seen on gfx950: an accumulator read two
// instructions after a 16x16x32 product on a taken-branch path); 24 wait
// states cover the longest (16-pass) products.  The scheduling barriers keep
// the products before and every reader after the padding.
__device__ __forceinline__ void mma_result_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  using T = uint16_t;
};
template <>
struct Elem<false> {
  using T = float;
};

template <bool BF16, int D>
struct KVFrag;
template <bool BF16, int D>
struct QFrag;

// ----------------------------------------------------------------- bf16 ---
template <int D>
struct KVFrag<true, D> {
  static constexpr int KS = D / 32;  // QK steps
  static constexpr int NT = D / 16;  // PV column tiles
  u32x4 k[KS];
  u32x2 v[NT];

  __device__ __forceinline__ void load_k(const uint16_t* kt, int lane) {
#pragma unroll
    for (int i = 0; i < KS; ++i) k[i] = *reinterpret_cast<const u32x4*>(kt + (i * kWave + lane) * 8);
  }
  __device__ __forceinline__ void load_v(const uint16_t* vt, int lane) {
    const int c = lane & 15, j = lane >> 4;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      v[t] = *reinterpret_cast<const u32x2*>(vt + (t * 16 + c) * kBlock + 4 * j);
  }
  __device__ __forceinline__ void load(const uint16_t* kt, const uint16_t* vt, int lane) {
    load_k(kt, lane);
    load_v(vt, lane);
  }
  __device__ __forceinline__ void zero_v() {
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = u32x2{0, 0};
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < KS; ++i) k[i] = u32x4{0, 0, 0, 0};
    zero_v();
  }
  // Zero the V entries of tokens 4j + r >= n_valid (tail slots of a block may
  // hold anything, NaN included; a zero weight times NaN would still be NaN).
  __device__ __forceinline__ void mask_v_tail(int n_valid, int lane) {
    const int t0 = 4 * (lane >> 4);
    const uint32_t lo = (t0 + 0 < n_valid ? 0x0000FFFFu : 0u) | (t0 + 1 < n_valid ? 0xFFFF0000u : 0u);
    const uint32_t hi = (t0 + 2 < n_valid ? 0x0000FFFFu : 0u) | (t0 + 3 < n_valid ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = u32x2{v[t].x & lo, v[t].y & hi};
  }
};

template <int D>
struct QFrag<true, D> {
  static constexpr int KS = D / 32;
  u32x4 q[KS];
  // row: the D elements of this lane's query row (lane & 15)
  __device__ __forceinline__ void load(const uint16_t* row, int lane) {
    const int j = lane >> 4;
#pragma unroll
    for (int i = 0; i < KS; ++i) q[i] = *reinterpret_cast<const u32x4*>(row + (4 * i + j) * 8);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < KS; ++i) q[i] = u32x4{0, 0, 0, 0};
  }
};

// S^T[token 4j + r][row c] = sum_d K[token][d] * Q[row][d]
template <int D>
__device__ __forceinline__ f32x4 qk_tile(const KVFrag<true, D>& f, const QFrag<true, D>& q) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KVFrag<true, D>::KS; i += 2) {
    s0 = mma_bf16_k32(f.k[i], q.q[i], s0);
    if (i + 1 < KVFrag<true, D>::KS) s1 = mma_bf16_k32(f.k[i + 1], q.q[i + 1], s1);
  }
  mma_result_fence();
  return s0 + s1;
}

// O[row 4j + r][16 t + c] += sum_k P[row][token k] V[token k][16 t + c]
template <int D>
__device__ __forceinline__ void pv_tile(f32x4 (&o)[D / 16], const float (&p)[4],
                                        const KVFrag<true, D>& f) {
  const u32x2 pa = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
#pragma unroll
  for (int t = 0; t < D / 16; ++t) o[t] = mma_bf16_k16(pa, f.v[t], o[t]);
}

// ----------------------------------------------------------------- fp32 ---
template <int D>
struct KVFrag<false, D> {
  static constexpr int KS = D / 16;  // 16-byte K chunks per lane (4 k-steps each)
  static constexpr int NT = D / 16;
  f32x4 k[KS];
  f32x4 v[NT];

  __device__ __forceinline__ void load_k(const float* kt, int lane) {
#pragma unroll
    for (int i = 0; i < KS; ++i) k[i] = *reinterpret_cast<const f32x4*>(kt + (i * kWave + lane) * 4);
  }
  __device__ __forceinline__ void load_v(const float* vt, int lane) {
    const int c = lane & 15, j = lane >> 4;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      v[t] = *reinterpret_cast<const f32x4*>(vt + (t * 16 + c) * kBlock + 4 * j);
  }
  __device__ __forceinline__ void load(const float* kt, const float* vt, int lane) {
    load_k(kt, lane);
    load_v(vt, lane);
  }
  __device__ __forceinline__ void zero_v() {
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < KS; ++i) k[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    zero_v();
  }
  __device__ __forceinline__ void mask_v_tail(int n_valid, int lane) {
    const int t0 = 4 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      v[t].x = (t0 + 0 < n_valid) ? v[t].x : 0.f;
      v[t].y = (t0 + 1 < n_valid) ? v[t].y : 0.f;
      v[t].z = (t0 + 2 < n_valid) ? v[t].z : 0.f;
      v[t].w = (t0 + 3 < n_valid) ? v[t].w : 0.f;
    }
  }
};

template <int D>
struct QFrag<false, D> {
  static constexpr int KS = D / 16;
  f32x4 q[KS];
  __device__ __forceinline__ void load(const float* row, int lane) {
    const int j = lane >> 4;
#pragma unroll
    for (int i = 0; i < KS; ++i) q[i] = *reinterpret_cast<const f32x4*>(row + (4 * i + j) * 4);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < KS; ++i) q[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// k-step (i, s) pairs dim 16 i + 4 j + s of K (A operand) and Q (B operand)
template <int D>
__device__ __forceinline__ f32x4 qk_tile(const KVFrag<false, D>& f, const QFrag<false, D>& q) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    s = mma_f32_k4(f.k[i].x, q.q[i].x, s);
    s = mma_f32_k4(f.k[i].y, q.q[i].y, s);
    s = mma_f32_k4(f.k[i].z, q.q[i].z, s);
    s = mma_f32_k4(f.k[i].w, q.q[i].w, s);
  }
  mma_result_fence();
  return s;
}

// k-step s pairs token 4 j + s of P (A operand) and V (B operand); P stays fp32
template <int D>
__device__ __forceinline__ void pv_tile(f32x4 (&o)[D / 16], const float (&p)[4],
                                        const KVFrag<false, D>& f) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    o[t] = mma_f32_k4(p[0], f.v[t].x, o[t]);
    o[t] = mma_f32_k4(p[1], f.v[t].y, o[t]);
    o[t] = mma_f32_k4(p[2], f.v[t].z, o[t]);
    o[t] = mma_f32_k4(p[3], f.v[t].w, o[t]);
  }
}

// Walk blocks 0 .. cnt-1 (cnt >= 1): fetch(buf, i) issues block i's loads and
// returns whether it is valid, step(buf, ok, i) consumes it.  With PREFETCH,
// block i + 1 is in flight while block i is computed (two register buffers);
// the steady-state loop always prefetches and the last one or two blocks are
// peeled off, so every path has the same loads outstanding and the compiler's
// wait counts stay exact.
template <bool PREFETCH, typename KV, typename Fetch, typename Step>
__device__ __forceinline__ void walk_blocks(int cnt, Fetch&& fetch, Step&& step) {
  if constexpr (PREFETCH) {
    KV bufA, bufB;
    bool okA = fetch(bufA, 0), okB;
    int i = 0;
    for (; i + 2 < cnt; i += 2) {
      okB = fetch(bufB, i + 1);
      step(bufA, okA, i);
      okA = fetch(bufA, i + 2);
      step(bufB, okB, i + 1);
    }
    if (i + 1 < cnt) {
      okB = fetch(bufB, i + 1);
      step(bufA, okA, i);
      step(bufB, okB, i + 1);
    } else {
      step(bufA, okA, i);
    }
  } else {
    for (int i = 0; i < cnt; ++i) {
      KV buf;
      const bool ok = fetch(buf, i);
      step(buf, ok, i);
    }
  }
}

// Walk blocks 0 .. cnt-1 (cnt >= 1) through a ring of NBUF register buffers:
// the loads of block i + NBUF - 1 are issued before block i is computed, so
// NBUF - 1 blocks stay in flight.  Loads are unconditional (past the end they
// re-read the last block, an L2 hit) so the compiler's wait counts stay exact;
// compute steps past the end are skipped.  Each refill waits out the wait
// states of the matrix ops that read the buffer last.
template <int NBUF, typename Buf, typename Fetch, typename Step>
__device__ __forceinline__ void walk_ring(int cnt, Fetch&& fetch, Step&& step) {
  Buf buf[NBUF];
  bool ok[NBUF];
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) ok[u] = fetch(buf[u], min(u, cnt - 1));
  for (int i = 0; i < cnt; i += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int nb = (u + NBUF - 1) % NBUF;
      mma_result_fence();
      ok[nb] = fetch(buf[nb], min(i + u + NBUF - 1, cnt - 1));
      if (i + u < cnt) step(buf[u], ok[u], i + u);
    }
  }
}

// Double-buffer unless two fragments would not fit the register file (fp32
// at head_dim 256: 128 registers per block).
template <bool BF16, int D>
constexpr bool kPrefetch = BF16 || D <= 128;

// Store 4 consecutive output elements.
__device__ __forceinline__ void store4(uint16_t* dst, f32x4 v) {
  *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
}
__device__ __forceinline__ void store4(float* dst, f32x4 v) { *reinterpret_cast<f32x4*>(dst) = v; }

__device__ __forceinline__ void store1(uint16_t* dst, float v) { *dst = (uint16_t)bf16_rne(v); }
__device__ __forceinline__ void store1(float* dst, float v) { *dst = v; }

// Raw logit -> base-2 logit (scale, optional softcap).
struct LogitXform {
  float scale_log2;  // scale * log2(e), used without softcap
  float scale;
  float cap;         // <= 0: off
  float inv_cap;
  __device__ __forceinline__ float operator()(float raw) const {
    return cap > 0.f ? softcap_log2(raw * scale, cap, inv_cap) : raw * scale_log2;
  }
};

__host__ __device__ inline LogitXform make_xform(float scale, float cap) {
  LogitXform x;
  x.scale_log2 = scale * 1.4426950408889634f;
  x.scale = scale;
  x.cap = cap;
  x.inv_cap = cap > 0.f ? 1.0f / cap : 0.f;
  return x;
}

}  // namespace pkv
