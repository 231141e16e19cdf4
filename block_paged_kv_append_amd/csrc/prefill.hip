// Causal chunked prefill over the block-paged cache.
//
// Pages: "Inference Server" (project README mirror), section "The engine" --
// prefill in chunks or batched, paged prefill kernels reading K/V through
// block tables, refcounted shared blocks; "Inference Server -- Architecture
// Map", section "How a single request flows through the system" -- a long
// prompt is prefilled one chunk per tick, after the cached prefix.
//
// Query rows are packed by GQA group: a matrix-core tile holds consecutive
// positions times the G query heads that share one kv head, so each K/V
// block loaded serves G heads at once.  A workgroup is one (sequence, kv
// head, range of positions) and walks every cache block its rows can see,
// running S^T = K Q^T and P V on the matrix cores with an online softmax per
// row.  Only blocks on the causal diagonal (or at a window edge) are partly
// masked; masking is by select.  Workgroups are numbered so that all ranges
// of one (sequence, kv head) land on the same XCD and share its L2.  Three
// forms:
//   * fp32 pools (prefill_kernel): 16-row tiles, blocks through registers;
//   * bf16 (prefill_pp_kernel): 32-row tiles on 32x32x16 products, stages of
//     32 keys streamed to LDS, two waves per SIMD sharing their rows and
//     splitting the stages (the prefill entry point);
//   * bf16, one wave per SIMD (prefill_mma32_body): the prefill part of the
//     one-launch mixed batch, whose decode workgroups run four waves.
#include <type_traits>

#include "attn_tile.hpp"
#include "launch.hpp"

#ifndef PKV_PREFILL_AHEAD
#define PKV_PREFILL_AHEAD 4
#endif
#ifndef PKV_PREFILL_RING
#define PKV_PREFILL_RING 4
#endif

namespace pkv {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));


template <bool BF16, int D, int RT>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a) {
  using T = typename Elem<BF16>::T;
  using KV = KVFrag<BF16, D>;
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  // wave index as a uniform (scalar) value: table lookups become scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, j = lane >> 4;
  const int G = a.gqa_group, Hkv = a.num_kv_heads, Hq = G * Hkv;
  const int PP = 16 / G;  // positions per row tile
  const LogitXform xf = make_xform(a.scale, a.softcap);

  // XCD-aware numbering: consecutive items (same sequence and kv head) go to
  // the same XCD (workgroups are dealt to the 8 XCDs round-robin).
  int item = blockIdx.x;
  if (a.num_items % 8 == 0) item = (blockIdx.x % 8) * (a.num_items / 8) + blockIdx.x / 8;
  const int tile = item % a.tiles_per_seq;
  const int bg = item / a.tiles_per_seq;
  const int g = bg % Hkv, b = bg / Hkv;

  const int L = min(max(a.context_lens[b], 0), a.max_blocks_per_seq * kBlock);
  const int r0 = min(max(a.cu_q_lens[b], 0), a.num_q_tokens);
  const int r1 = min(max(a.cu_q_lens[b + 1], r0), a.num_q_tokens);
  const int n = r1 - r0;
  const int pos_wave = tile * (kWaves * RT * PP) + wave * RT * PP;
  if (pos_wave >= n) return;
  const int shift = L - n;  // position j of the chunk sits at token shift + j

  QFrag<BF16, D> qf[RT];
  int qpos[RT];     // query position of this lane's row c in tile t
  bool rvalid[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int pos = pos_wave + t * PP + c / G;
    rvalid[t] = pos < n;
    qpos[t] = shift + pos;
    if (rvalid[t])
      qf[t].load(reinterpret_cast<const T*>(a.q) + ((size_t)(r0 + pos) * Hq + g * G + c % G) * D,
                 lane);
    else
      qf[t].zero();
  }

  const int p_hi = min(n - 1, pos_wave + RT * PP - 1);
  const int last_tok = min(shift + p_hi, L - 1);
  const int first_tok = a.window > 0 ? max(0, shift + pos_wave - a.window + 1) : 0;
  if (last_tok < 0) {
    // every row of this wave sits before the cache (a chunk longer than its
    // context, a caller error): no key is visible, out = 0 and lse = -inf
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int pos = pos_wave + t * PP + c / G;
      if (pos >= n) continue;
      const size_t row = (size_t)(r0 + pos) * Hq + g * G + c % G;
      if (a.lse != nullptr && j == 0) a.lse[row] = kNegInf;
      T* dst = reinterpret_cast<T*>(a.out) + row * D;
      for (int d = j; d < D; d += 4) store1(dst + d, 0.f);
    }
    return;
  }
  const int blk_lo = first_tok / kBlock, blk_hi = last_tok / kBlock;

  f32x4 o[RT][NT];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    m_run[t] = kNegInf;
    l_run[t] = 0.f;
#pragma unroll
    for (int x = 0; x < NT; ++x) o[t][x] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  const T* kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* vpool = reinterpret_cast<const T*>(a.v_pool);
  constexpr size_t kTile = (size_t)D * kBlock;

  // Table entries of blocks blk_lo .. blk_hi, 64 at a time, one per lane;
  // loads are unconditional (an out-of-range entry reads block 0 and is masked
  // out) so that every path keeps the same loads in flight.
  int tbl = 0, tbl_base = blk_lo;
  auto fetch = [&](KV& buf, int blk) -> bool {
    const int phys = __builtin_amdgcn_readlane(tbl, (blk - tbl_base) & 63);
    const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
    const size_t off = ((size_t)(ok ? phys : 0) * Hkv + g) * kTile;
    buf.load(kpool + off, vpool + off, lane);
    return ok;
  };

  auto step = [&](KV& buf, bool ok, int blk) {
    const int tok0 = blk * kBlock;
    if (!ok)
      buf.zero();
    else if (tok0 + kBlock > L)
      buf.mask_v_tail(L - tok0, lane);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const f32x4 sc = qk_tile<D>(buf, qf[t]);
      float s2[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tk = tok0 + 4 * j + r;
        const bool vis = ok & rvalid[t] & (tk < L) & (tk <= qpos[t]) &
                         ((a.window <= 0) | (qpos[t] - tk < a.window));
        s2[r] = vis ? xf(sc[r]) : kNegInf;
      }
      float mx = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[t], mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[t] - m_use);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s2[r] - m_use);
      l_run[t] = l_run[t] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
      m_run[t] = m_new;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * j + r);
#pragma unroll
      for (int x = 0; x < NT; ++x) {
        o[t][x].x *= ar[0];
        o[t][x].y *= ar[1];
        o[t][x].z *= ar[2];
        o[t][x].w *= ar[3];
      }
      pv_tile<D>(o[t], p, buf);
    }
  };

  for (tbl_base = blk_lo; tbl_base <= blk_hi; tbl_base += 64) {
    const int cnt = min(64, blk_hi - tbl_base + 1);
    tbl = lane < cnt ? bt[tbl_base + lane] : 0;
    walk_blocks<kPrefetch<BF16, D>, KV>(
        cnt, [&](KV& buf, int i) { return fetch(buf, tbl_base + i); },
        [&](KV& buf, bool ok, int i) { step(buf, ok, tbl_base + i); });
  }

  // ---- finalize: rows 4j + r of each tile ----
  mma_result_fence();
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    float l_tot = l_run[t] + __shfl_xor(l_run[t], 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (a.lse != nullptr && j == 0) {
      const int pos = pos_wave + t * PP + c / G;
      if (pos < n)
        a.lse[(size_t)(r0 + pos) * Hq + g * G + c % G] =
            l_tot > 0.f ? (m_run[t] + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * j + r;
      const float lr = __shfl(l_tot, m);
      const int pos = pos_wave + t * PP + m / G;
      if (pos >= n) continue;
      const float inv = lr > 0.f ? 1.0f / lr : 0.f;
      T* dst = reinterpret_cast<T*>(a.out) + ((size_t)(r0 + pos) * Hq + g * G + m % G) * D + c;
#pragma unroll
      for (int x = 0; x < NT; ++x) store1(dst + x * 16, o[t][x][r] * inv);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 form on 32x32x16 matrix-core tiles.
//
// A wave owns 32 GQA-packed query rows (32 / G positions times G heads); the
// four waves of a workgroup cover consecutive positions of one (sequence, kv
// head).  Keys are taken 32 at a time (two cache blocks, a "stage"):
//   S^T[32 keys][32 rows] = K Q^T         (D/16 products, k = 16 dims)
//   O^T[D][32 rows]      += V^T P^T       (D/32 row tiles x 2 blocks, k = 16 keys)
// Computing O transposed keeps a row's statistics (max, sum, rescale factor)
// in the two lanes that hold that row's scores, so the softmax needs one
// cross-half lane swap per stage and no other exchange.
//
// K/V reach LDS by direct global->LDS copies (16 bytes per lane, a wave
// writes 1 KiB contiguous, each lane picks its own source).  The copy lays
// every stage out in the order the matrix cores consume it, so each operand
// is one linear 1 KiB LDS read:
//   K run s (s < D/16): lane (i, kg) <- K[block i/16][token pi(i%16)][dims 16s + 8kg .. +7]
//   V run 2x+q:         lane (i, kg) <- V[block q][tokens 8kg .. +7][dim 32x + i]
// where pi swaps bits 2 and 3 of the token index, which makes the score tile's
// register v of lane (n, kg) the score of key 16*(v/8) + 8kg + v%8: the same
// lane then holds, per block, exactly the 8 probabilities the V^T P^T product
// wants from it.  NB stage buffers form a ring; copies run NB-2 stages ahead
// and each stage costs one barrier.  The next stage's S^T is computed before
// the current stage's softmax and P V, so matrix-core and vector work overlap.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0) only
}
// Issue order for a region of NMF matrix-core products fed by NMF LDS
// operand reads: the reads run four products ahead, NVA vector
// instructions sit in each product's shadow.
template <int NMF, int NVA>
__device__ __forceinline__ void pipeline_order() {
  constexpr int kAhead = NMF < 4 ? NMF : 4;
  __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
  for (int i = 0; i < NMF - kAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NVA, 0);
  }
#pragma unroll
  for (int i = 0; i < kAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NVA, 0);
  }
}
// buffer resource of one block's K (or V) tile: a raw byte range, empty when
// the block may not be read (copies then return zeros)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
  constexpr unsigned kRawBufferWord3 = 0x00020000u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRawBufferWord3);
}
// 16 bytes per lane from the buffer into LDS; a wave writes 1 KiB starting at
// wave_dst, lane i at +16 i.  A buffer (not global) copy: the compiler's LDS
// wait counting stays exact around it.
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t r, int byte_off, uint32_t sbyte_off,
                                            u32x4* wave_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)wave_dst, 16, byte_off,
                                           (int)sbyte_off, 0, 0);
}

// LDS of the matrix-core prefill: NB stages of K and V runs
template <int D, int NB>
constexpr int kPrefillStageU4 = (D / 16 + 2 * (D / 32)) * kWave;
template <int D, int NB>
constexpr size_t kPrefillLdsBytes = (size_t)NB * kPrefillStageU4<D, NB> * 16;

// The prefill of work item `blk` (before the XCD-aware renumbering), with
// `smem` its stage ring in LDS, by four waves: the mixed-batch kernel runs it
// for the first workgroups of its grid.
template <int D, int NB, bool SC, bool FLAT>
__device__ __forceinline__ void prefill_mma32_body(const PrefillArgs& a, int blk, u32x4* smem) {
  constexpr int KD = D / 16;                    // K runs per stage = QK products
  constexpr int XT = D / 32;                    // output row tiles of O^T
  constexpr int kRuns = KD + 2 * XT;            // 1 KiB runs per stage
  constexpr int kStageU4 = kRuns * kWave;       // 16-byte chunks per stage
  constexpr int kDma = kRuns / kWaves;          // copies per wave per stage
  static_assert(kDma * 2 == 2 * XT, "one copy every second P V product");
  constexpr int kAhead = PKV_PREFILL_AHEAD;     // LDS operand reads in flight
  constexpr int kTileU4 = D * kBlock * 2 / 16;  // chunks of one block's K (or V) in the pool
  static_assert(KD % kWaves == 0 && (2 * XT) % kWaves == 0, "runs must split over the waves");
  static_assert(NB >= 3 && (NB & (NB - 1)) == 0, "ring of 4 or 8 stages");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, kg = lane >> 5;
  const int G = a.gqa_group, Hkv = a.num_kv_heads, Hq = G * Hkv;
  const int PPW = 32 / G;  // positions per wave
  const LogitXform xf = make_xform(a.scale, a.softcap);
  // Scores are masked to -inf before the logit transform.  Without softcap
  // that transform is one multiply, which must keep -inf: the factor is made
  // positive by flipping the sign of q for a negative scale, and a zero scale
  // becomes a tiny positive factor (-inf * 0 would be NaN).
  const bool flip_q = !SC && xf.scale_log2 < 0.f;
  const float pos_scale_log2 = fmaxf(fabsf(xf.scale_log2), 1e-30f);

  int item = blk;
  if (a.num_items % 8 == 0) item = (int)((unsigned)blk % 8u) * (a.num_items / 8) + (int)((unsigned)blk / 8u);
  const int tile = item % a.tiles_per_seq;
  const int bg = item / a.tiles_per_seq;
  const int g = bg % Hkv, b = bg / Hkv;

  const int L = min(max(a.context_lens[b], 0), a.max_blocks_per_seq * kBlock);
  const int r0 = min(max(a.cu_q_lens[b], 0), a.num_q_tokens);
  const int r1 = min(max(a.cu_q_lens[b + 1], r0), a.num_q_tokens);
  const int nq = r1 - r0;
  const int pos_wg = tile * (kWaves * PPW);
  if (pos_wg >= nq) return;  // whole workgroup, before any barrier
  const int shift = L - nq;
  const int pos_wave = pos_wg + wave * PPW;
  const bool wave_live = pos_wave < nq;
  const int pos = pos_wave + n / G;
  const bool rvalid = pos < nq;
  const int qpos = shift + pos;
  const int head = g * G + n % G;
  // positions of the wave's first and last real row (uniform)
  const int qpos_lo = shift + pos_wave;
  const int qpos_hi = shift + min(pos_wave + PPW - 1, nq - 1);

  u32x4 qf[KD];
  {
    const uint16_t* row =
        reinterpret_cast<const uint16_t*>(a.q) + ((size_t)(r0 + min(pos, nq - 1)) * Hq + head) * D + 8 * kg;
#pragma unroll
    for (int i = 0; i < KD; ++i) qf[i] = *reinterpret_cast<const u32x4*>(row + 16 * i);
    if (flip_q) {
      const uint32_t sgn = 0x80008000u;  // both bf16 halves of each word
#pragma unroll
      for (int i = 0; i < KD; ++i) qf[i] ^= u32x4{sgn, sgn, sgn, sgn};
    }
    // the query fragments live in the accumulator file (the matrix cores
    // read operands from either file), leaving vector registers for operand
    // prefetch
#pragma unroll
    for (int i = 0; i < KD; ++i) asm volatile("" : "=a"(qf[i]) : "0"(qf[i]));
  }

  // keys the workgroup's rows can see
  const int p_hi = min(nq - 1, pos_wg + kWaves * PPW - 1);
  const int last_tok = min(shift + p_hi, L - 1);
  if (last_tok < 0) {
    // every row of the workgroup sits before the cache (a chunk longer than
    // its context, a caller error): no key is visible, out = 0, lse = -inf
    if (wave_live && rvalid) {
      const size_t row = (size_t)(r0 + pos) * Hq + head;
      if (a.lse != nullptr && kg == 0) a.lse[row] = kNegInf;
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + row * D + 4 * kg;
#pragma unroll
      for (int x = 0; x < D / 8; ++x) *reinterpret_cast<u32x2*>(dst + 8 * x) = u32x2{0u, 0u};
    }
    return;
  }
  const int first_tok = a.window > 0 ? max(0, shift + pos_wg - a.window + 1) : 0;
  const int blk_lo = first_tok / kBlock;
  const int nblk = last_tok / kBlock - blk_lo + 1;
  const int nstage = (nblk + 1) / 2;
  const int* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq + blk_lo;
  const u32x4* kpool = reinterpret_cast<const u32x4*>(a.k_pool);
  const u32x4* vpool = reinterpret_cast<const u32x4*>(a.v_pool);

  // per-lane chunk offsets of the copies within a block (see the layout above)
  const int k_off = 16 * (lane >> 4) + ((lane & 3) | ((lane & 4) << 1) | ((lane & 8) >> 1));
  const int v_off = 2 * n + kg;
  // where lane (n, kg) finds its K operand inside a pair of runs
  const int k_rd = ((n >> 4) << 6) + (n & 15) + 16 * kg;

  // Block-table entries, 64 per vector register (lane i: entry base + i),
  // the next slice loaded one slice ahead; read out with a lane select.
  int tbl_cur = lane < nblk ? bt[lane] : 0;
  int tbl_nxt = 64 + lane < nblk ? bt[64 + lane] : 0;
  int tbl_base = 0;
  uint32_t okbits = 0;    // bit 2 * (stage % NB) + q: block q of that stage is readable
  uint32_t fullbits = 0;  // bit stage % NB: every score visible to every real row of the wave
  uint32_t tailbits = 0;  // bit stage % NB: some key of the stage is past the context or unreadable
  // Copies of one stage: descriptors made once (prepare), the copies issued
  // one every second product of the next P V phase (copy); in one burst
  // they would hold the waves on the vector memory path.  A wave copies the
  // runs of one block of the stage, block (wave & 1).  FLAT (each pool under
  // 4 GiB): one descriptor per pool for the whole call, and per stage only
  // the byte offset of the wave's block (an unreadable block reads block 0,
  // whose keys are masked and whose values are cleared like a tail's);
  // otherwise a descriptor per block, empty for an unreadable one.
  __amdgpu_buffer_rsrc_t crk0, crk1, crv0, crv1;
  uint32_t csoff = 0;
  const __amdgpu_buffer_rsrc_t rkp =
      tile_rsrc(kpool, FLAT ? (int)(uint32_t)((size_t)a.num_blocks * Hkv * kTileU4 * 16) : 0);
  const __amdgpu_buffer_rsrc_t rvp =
      tile_rsrc(vpool, FLAT ? (int)(uint32_t)((size_t)a.num_blocks * Hkv * kTileU4 * 16) : 0);
  u32x4* cdst = smem;
  auto prepare = [&](int st) {
    if (2 * st - tbl_base >= 64) {  // uniform, every 32 stages
      tbl_base += 64;
      tbl_cur = tbl_nxt;
      tbl_nxt = tbl_base + 64 + lane < nblk ? bt[tbl_base + 64 + lane] : 0;
    }
    const int cur[2] = {__builtin_amdgcn_readlane(tbl_cur, 2 * st - tbl_base),
                        __builtin_amdgcn_readlane(tbl_cur, 2 * st + 1 - tbl_base)};
    uint32_t ok2 = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int lb = 2 * st + q;
      const bool ok = lb < nblk && (unsigned)cur[q] < (unsigned)a.num_blocks;
      ok2 |= (uint32_t)ok << q;
      if constexpr (!FLAT) {
        const size_t off = ((size_t)(ok ? cur[q] : 0) * Hkv + g) * kTileU4;
        // an unreadable block gets an empty range: its copies read zeros
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kpool + off, ok ? kTileU4 * 16 : 0);
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vpool + off, ok ? kTileU4 * 16 : 0);
        if (q == 0) {
          crk0 = rk;
          crv0 = rv;
        } else {
          crk1 = rk;
          crv1 = rv;
        }
      }
    }
    if constexpr (FLAT) {
      const int q = wave & 1;  // the block this wave copies
      const int ph = q ? cur[1] : cur[0];
      csoff = ((ok2 >> q) & 1u) ? (uint32_t)(ph * Hkv + g) * (uint32_t)(kTileU4 * 16) : 0u;
    }
    const int tok0 = (blk_lo + 2 * st) * kBlock;
    const bool full = ok2 == 3u && tok0 + 31 < L && tok0 + 31 <= qpos_lo &&
                      (a.window <= 0 || qpos_hi - tok0 < a.window);
    const bool tail = !(ok2 == 3u && tok0 + 2 * kBlock <= L);
    const int slot = st & (NB - 1);
    okbits = (okbits & ~(3u << (2 * slot))) | (ok2 << (2 * slot));
    fullbits = (fullbits & ~(1u << slot)) | ((uint32_t)full << slot);
    tailbits = (tailbits & ~(1u << slot)) | ((uint32_t)tail << slot);
    cdst = smem + slot * kStageU4;
  };
  // This wave's copy j of the prepared stage.  K runs 2p, 2p+1 form 2 KiB:
  // the first KiB from block 0 (run 2p's lanes n < 16, then run 2p+1's),
  // the second from block 1; each copy reads one block.
  // With per-block descriptors (pools over 4 GiB) a copy's 1 KiB run offset
  // goes to the scalar offset, so that all of a wave's copies share one
  // lane-offset register for K and one for V: the descriptors take registers
  // the loop would otherwise spill for.
  const int k_lane = k_off * 16, v_lane = v_off * 16;
  auto copy = [&](int j) {
    if (j < KD / kWaves) {
      const int pr = 2 * j + (wave >> 1);
      u32x4* dst = cdst + pr * 2 * kWave + (wave & 1) * kWave;
      if constexpr (FLAT)
        copy_to_lds(rkp, (64 * pr + k_off) * 16, csoff, dst);
      else
        copy_to_lds((wave & 1) ? crk1 : crk0, k_lane, pr * 1024, dst);
    } else {
      const int x = 2 * (j - KD / kWaves) + (wave >> 1);
      u32x4* dst = cdst + (KD + 2 * x + (wave & 1)) * kWave;
      if constexpr (FLAT)
        copy_to_lds(rvp, (64 * x + v_off) * 16, csoff, dst);
      else
        copy_to_lds((wave & 1) ? crv1 : crv0, v_lane, x * 1024, dst);
    }
  };
  auto issue = [&](int st) {
    prepare(st);
#pragma unroll
    for (int j = 0; j < kDma; ++j) copy(j);
  };

  // chunk offset of K run s within a stage, relative to k_rd
  auto k_run = [](int s) { return (s >> 1) * 2 * kWave + (s & 1) * 32; };
  auto stage_tok0 = [&](int st) { return (blk_lo + 2 * st) * kBlock; };
  auto stage_ok = [&](int st) { return (okbits >> (2 * (st & (NB - 1)))) & 3u; };
  auto stage_full = [&](int st) { return (fullbits >> (st & (NB - 1))) & 1u; };
  // Keys past the context (or of an unreadable block) may hold anything; in
  // LDS their V entries are cleared once the stage has landed, so that the
  // products never multiply a zero probability by a non-finite value.  Rare
  // (the context's last block), done by the whole workgroup.
  auto clear_v_tail = [&](int st) {
    if (!((tailbits >> (st & (NB - 1))) & 1u)) return;
    const int tok0 = stage_tok0(st);
    const uint32_t okk = stage_ok(st);
    u32x4* vr = smem + (st & (NB - 1)) * kStageU4 + KD * kWave;
    for (int c = threadIdx.x; c < 2 * XT * kWave; c += kThreads) {
      const int q = (c >> 6) & 1, kgc = (c >> 5) & 1;
      const int nv = ((okk >> q) & 1u) ? L - (tok0 + 16 * q) - 8 * kgc : 0;
      if (nv >= 8) continue;
      const u32x4 m = {(0 < nv ? 0x0000FFFFu : 0u) | (1 < nv ? 0xFFFF0000u : 0u),
                       (2 < nv ? 0x0000FFFFu : 0u) | (3 < nv ? 0xFFFF0000u : 0u),
                       (4 < nv ? 0x0000FFFFu : 0u) | (5 < nv ? 0xFFFF0000u : 0u),
                       (6 < nv ? 0x0000FFFFu : 0u) | (7 < nv ? 0xFFFF0000u : 0u)};
      vr[c] = vr[c] & m;
    }
    wait_lds();  // written before this wave reaches the next barrier
  };
  // score (raw S^T element v of stage st) -> -inf where not visible
  auto mask_scores = [&](int st, f32x16& sc) {
    const int tok0 = stage_tok0(st);
    const uint32_t okk = stage_ok(st);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tk = tok0 + 16 * (v >> 3) + 8 * kg + (v & 7);
      const bool vis = ((okk >> (v >> 3)) & 1u) & rvalid & (tk < L) & (tk <= qpos) &
                       ((a.window <= 0) | (qpos - tk < a.window));
      sc[v] = vis ? sc[v] : kNegInf;
    }
  };
  // base-2 logit; a masked score stays -inf
  auto logit = [&](float x) {
    if constexpr (SC) {
      const float y = softcap_log2(x * xf.scale, xf.cap, xf.inv_cap);
      return x == kNegInf ? kNegInf : y;
    } else {
      return x * pos_scale_log2;
    }
  };

  f32x16 o[XT];
#pragma unroll
  for (int x = 0; x < XT; ++x) o[x] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  constexpr float kLazy = 8.0f;  // rescale only when the max grows by 2^8
  float sv[16];                  // base-2 logits of the stage to exponentiate next

  // new row maxima: grow the running max (rarely) and rescale what is summed
  auto update_max = [&]() {
    float mx = sv[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sv[v]);
    mx = half_max(mx);
    if (__any(mx > m_run + kLazy)) {
      mma_result_fence();
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int x = 0; x < XT; ++x) o[x] *= alpha;
      m_run = m_new;
    }
  };

#pragma unroll
  for (int st = 0; st < NB - 1; ++st) issue(st);
  wait_vmem<(NB - 2) * kDma>();
  lds_barrier();
  clear_v_tail(0);
  lds_barrier();
  if (wave_live) {
    const u32x4* kb = smem + k_rd;
    f32x16 acc = {};
#pragma unroll
    for (int i = 0; i < KD; ++i) acc = mma32_bf16(kb[k_run(i)], qf[i], acc);
    mma_result_fence();
    if (!stage_full(0)) mask_scores(0, acc);
#pragma unroll
    for (int v = 0; v < 16; ++v) sv[v] = logit(acc[v]);
    update_max();
  }

  // Stage k, in two phases without branches:
  //   1: S^T of stage k + 1 on the matrix cores  |  exponentials of stage k
  //   2: O^T += V^T P^T of stage k               |  logits and max of stage k + 1
  // Operand reads run up to four products ahead of their use.  The last trip
  // computes the scores of a dummy stage: fully masked, never used.
  for (int k = 0; k < nstage; ++k) {
    wait_vmem<(NB - 3) * kDma>();  // stage k + 1 has landed (this wave's part)
    lds_barrier();                 // ... and every other wave's
    if (k + 1 < nstage) clear_v_tail(k + 1);
    prepare(k + NB - 1);  // into the slot stage k - 1 used
    if (!wave_live) {
#pragma unroll
      for (int j = 0; j < kDma; ++j) copy(j);
      continue;
    }

    // phase 1: the order below is the issue order (scheduling barriers)
    constexpr int kE = 16 / KD;  // score elements handled per product
    const u32x4* kb = smem + ((k + 1) & (NB - 1)) * kStageU4 + k_rd;
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    f32x16 acc = {};
    float p[16];
    uint32_t pw[8];  // probabilities as bf16 pairs
    float ls = 0.f;
    {
      u32x4 kf[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead && i < KD; ++i) kf[i] = kb[k_run(i)];
#pragma unroll
      for (int i = 0; i < KD; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        acc = mma32_bf16(kf[i % kAhead], qf[i], acc);
        if (i + kAhead < KD) kf[i % kAhead] = kb[k_run(i + kAhead)];
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          const int v = i * kE + e;
          p[v] = fast_exp2(sv[v] - m_use);
          ls += p[v];
          if (v & 1) pw[v >> 1] = pack_bf16x2_hw(p[v - 1], p[v]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    l_run += ls;
    const u32x4 pb[2] = {u32x4{pw[0], pw[1], pw[2], pw[3]}, u32x4{pw[4], pw[5], pw[6], pw[7]}};
    asm volatile("" ::"v"(pb[0]), "v"(pb[1]), "v"(l_run));  // computed here, not sunk into phase 2

    mma_result_fence();
    if (!stage_full(k + 1)) mask_scores(k + 1, acc);

    // phase 2
    const u32x4* vb = smem + (k & (NB - 1)) * kStageU4 + KD * kWave + lane;
    {
      constexpr int NU = 2 * XT;  // products: u = q * XT + x
      u32x4 vf[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead && u < NU; ++u) vf[u] = vb[(2 * (u % XT) + u / XT) * kWave];
      float mx = kNegInf;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        const int x = u % XT, q = u / XT;
        o[x] = mma32_bf16(vf[u % kAhead], pb[q], o[x]);
        if (u + kAhead < NU) vf[u % kAhead] = vb[(2 * ((u + kAhead) % XT) + (u + kAhead) / XT) * kWave];
        if ((u & 1) == 0) copy(u >> 1);  // kDma = NU / 2 copies
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          sv[u * kE + e] = logit(acc[u * kE + e]);
          mx = fmaxf(mx, sv[u * kE + e]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      mx = half_max(mx);
      if (__any(mx > m_run + kLazy)) {
        mma_result_fence();
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
        l_run *= alpha;
#pragma unroll
        for (int x2 = 0; x2 < XT; ++x2) o[x2] *= alpha;
        m_run = m_new;
      }
    }
  }
  wait_vmem<0>();  // no copy may still be in flight when the workgroup ends
  mma_result_fence();
  if (!wave_live) return;

  const float l_tot = half_sum(l_run);
  if (a.lse != nullptr && kg == 0 && rvalid)
    a.lse[(size_t)(r0 + pos) * Hq + head] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  if (!rvalid) return;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + ((size_t)(r0 + pos) * Hq + head) * D + 4 * kg;
#pragma unroll
  for (int x = 0; x < XT; ++x)
#pragma unroll
    for (int h = 0; h < 4; ++h)
      *reinterpret_cast<u32x2*>(dst + 32 * x + 8 * h) =
          u32x2{pack_bf16x2_hw(o[x][4 * h] * inv, o[x][4 * h + 1] * inv),
                pack_bf16x2_hw(o[x][4 * h + 2] * inv, o[x][4 * h + 3] * inv)};
}

// ---------------------------------------------------------------------------
// Two waves per SIMD ("ping-pong").  With one wave per SIMD, the vector work
// of a stage (softmax, masking, addressing) issues mostly outside the
// matrix-core products' shadow: a single wave hides only about two vector
// instructions under each 32x32x16 product.  Here a workgroup has eight
// waves; waves w and w + 4 share a SIMD and the same 32 query rows, and take
// alternate stages (w < 4 the even ones, w >= 4 the odd ones), each with its
// own online softmax over its stages.  While one wave of a pair is in its
// softmax, the other's products keep the matrix core busy.  Each wave runs a
// stage in order (S^T, softmax, P V), so no second score tile is live, and
// the pair's two partial results are merged by log-sum-exp through LDS at
// the end, each wave writing half of the output dims.
//
// Stages move through the same NB-slot LDS ring as above, one "interval"
// (two stages, one per half) per barrier: at the barrier of interval i,
// stages 2i and 2i + 1 have landed and every wave has finished interval
// i - 1, so the copies of interval i + NB/2 - 1 go into the slots interval
// i - 1 used.  Each half copies its own parity's stages, split over its four
// waves exactly as in the four-wave form.
template <int D, int NB>
constexpr size_t kPrefillPPLdsBytes =
    (size_t)NB * kPrefillStageU4<D, NB> * 16 > (size_t)8 * ((D / 64) * 16 * kWave + 2 * kWave) * 4
        ? (size_t)NB * kPrefillStageU4<D, NB> * 16
        : (size_t)8 * ((D / 64) * 16 * kWave + 2 * kWave) * 4;

template <int D, int NB, bool SC, bool FLAT>
__device__ __forceinline__ void prefill_pp_body(const PrefillArgs& a, int blk, u32x4* smem) {
  constexpr int KD = D / 16;                    // K runs per stage = QK products
  constexpr int XT = D / 32;                    // output row tiles of O^T
  constexpr int kRuns = KD + 2 * XT;            // 1 KiB runs per stage
  constexpr int kStageU4 = kRuns * kWave;       // 16-byte chunks per stage
  constexpr int kDma = kRuns / kWaves;          // copies per wave per interval
  constexpr int kAhead = D >= 256 ? 2 : 4;      // LDS operand reads in flight (registers)
  constexpr int kTileU4 = D * kBlock * 2 / 16;  // chunks of one block's K (or V) in the pool
  constexpr int kAheadIv = NB / 2 - 1;          // intervals the copies run ahead
  static_assert(KD == 2 * kDma, "one copy every second S^T product");
  static_assert(NB >= 4 && (NB & (NB - 1)) == 0, "ring of 4 or 8 stages");
  static_assert(XT % 2 == 0, "output tiles split between the pair");

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = w & 3;  // row group (and copy share within a half)
  const int half = w >> 2; // stage parity
  const int n = lane & 31, kg = lane >> 5;
  const int G = a.gqa_group, Hkv = a.num_kv_heads, Hq = G * Hkv;
  const int PPW = 32 / G;
  const LogitXform xf = make_xform(a.scale, a.softcap);
  const bool flip_q = !SC && xf.scale_log2 < 0.f;
  const float pos_scale_log2 = fmaxf(fabsf(xf.scale_log2), 1e-30f);

#ifdef PKV_TIMELINE
  // timeline build: shader-clock and real-time counters at entry and exit
  unsigned long long tl_cyc0 = 0, tl_rt0 = 0;
  if (threadIdx.x == 0) {
    tl_cyc0 = __builtin_amdgcn_s_memtime();
    tl_rt0 = __builtin_amdgcn_s_memrealtime();
  }
#endif
  int item = blk;
  if (a.num_items % 8 == 0) item = (int)((unsigned)blk % 8u) * (a.num_items / 8) + (int)((unsigned)blk / 8u);
  const int tile = item % a.tiles_per_seq;
  const int bg = item / a.tiles_per_seq;
  const int g = bg % Hkv, b = bg / Hkv;

  const int L = min(max(a.context_lens[b], 0), a.max_blocks_per_seq * kBlock);
  const int r0 = min(max(a.cu_q_lens[b], 0), a.num_q_tokens);
  const int r1 = min(max(a.cu_q_lens[b + 1], r0), a.num_q_tokens);
  const int nq = r1 - r0;
  const int pos_wg = tile * (kWaves * PPW);
  if (pos_wg >= nq) return;  // whole workgroup, before any barrier
  const int shift = L - nq;
  const int pos_wave = pos_wg + wave * PPW;
  const bool wave_live = pos_wave < nq;
  const int pos = pos_wave + n / G;
  const bool rvalid = pos < nq;
  const int qpos = shift + pos;
  const int head = g * G + n % G;
  const int qpos_lo = shift + pos_wave;
  const int qpos_hi = shift + min(pos_wave + PPW - 1, nq - 1);

  const int p_hi = min(nq - 1, pos_wg + kWaves * PPW - 1);
  const int last_tok = min(shift + p_hi, L - 1);
  if (last_tok < 0) {
    // every row of the workgroup sits before the cache: out = 0, lse = -inf
    if (half == 0 && wave_live && rvalid) {
      const size_t row = (size_t)(r0 + pos) * Hq + head;
      if (a.lse != nullptr && kg == 0) a.lse[row] = kNegInf;
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + row * D + 4 * kg;
#pragma unroll
      for (int x = 0; x < D / 8; ++x) *reinterpret_cast<u32x2*>(dst + 8 * x) = u32x2{0u, 0u};
    }
    return;
  }

  u32x4 qf[KD];
  {
    const uint16_t* row =
        reinterpret_cast<const uint16_t*>(a.q) + ((size_t)(r0 + min(pos, nq - 1)) * Hq + head) * D + 8 * kg;
#pragma unroll
    for (int i = 0; i < KD; ++i) qf[i] = *reinterpret_cast<const u32x4*>(row + 16 * i);
    if (flip_q) {
      const uint32_t sgn = 0x80008000u;
#pragma unroll
      for (int i = 0; i < KD; ++i) qf[i] ^= u32x4{sgn, sgn, sgn, sgn};
    }
    // the query fragments stay in vector registers: with two waves per SIMD
    // a wave has 256 registers, and using the accumulator file at all would
    // split them evenly between the two files
  }

  const int first_tok = a.window > 0 ? max(0, shift + pos_wg - a.window + 1) : 0;
  const int blk_lo = first_tok / kBlock;
  const int nblk = last_tok / kBlock - blk_lo + 1;
  const int nstage = (nblk + 1) / 2;
  const int n_iv = (nstage + 1) / 2;
  const int* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq + blk_lo;
  const u32x4* kpool = reinterpret_cast<const u32x4*>(a.k_pool);
  const u32x4* vpool = reinterpret_cast<const u32x4*>(a.v_pool);

  const int k_off = 16 * (lane >> 4) + ((lane & 3) | ((lane & 4) << 1) | ((lane & 8) >> 1));
  const int v_off = 2 * n + kg;
  const int k_rd = ((n >> 4) << 6) + (n & 15) + 16 * kg;

  // block-table slices and per-slot stage flags, as in the four-wave form;
  // a wave prepares (and later computes) only the stages of its parity
  int tbl_cur = lane < nblk ? bt[lane] : 0;
  int tbl_nxt = 64 + lane < nblk ? bt[64 + lane] : 0;
  int tbl_base = 0;
  uint32_t okbits = 0, fullbits = 0, tailbits = 0;
  __amdgpu_buffer_rsrc_t crk0, crk1, crv0, crv1;
  uint32_t csoff = 0;
  const __amdgpu_buffer_rsrc_t rkp =
      tile_rsrc(kpool, FLAT ? (int)(uint32_t)((size_t)a.num_blocks * Hkv * kTileU4 * 16) : 0);
  const __amdgpu_buffer_rsrc_t rvp =
      tile_rsrc(vpool, FLAT ? (int)(uint32_t)((size_t)a.num_blocks * Hkv * kTileU4 * 16) : 0);
  u32x4* cdst = smem;
  auto prepare = [&](int st) {
    while (2 * st - tbl_base >= 64) {  // uniform
      tbl_base += 64;
      tbl_cur = tbl_nxt;
      tbl_nxt = tbl_base + 64 + lane < nblk ? bt[tbl_base + 64 + lane] : 0;
    }
    const int cur[2] = {__builtin_amdgcn_readlane(tbl_cur, 2 * st - tbl_base),
                        __builtin_amdgcn_readlane(tbl_cur, 2 * st + 1 - tbl_base)};
    uint32_t ok2 = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int lb = 2 * st + q;
      const bool ok = lb < nblk && (unsigned)cur[q] < (unsigned)a.num_blocks;
      ok2 |= (uint32_t)ok << q;
      if constexpr (!FLAT) {
        const size_t off = ((size_t)(ok ? cur[q] : 0) * Hkv + g) * kTileU4;
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kpool + off, ok ? kTileU4 * 16 : 0);
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vpool + off, ok ? kTileU4 * 16 : 0);
        if (q == 0) {
          crk0 = rk;
          crv0 = rv;
        } else {
          crk1 = rk;
          crv1 = rv;
        }
      }
    }
    if constexpr (FLAT) {
      const int q = wave & 1;
      const int ph = q ? cur[1] : cur[0];
      csoff = ((ok2 >> q) & 1u) ? (uint32_t)(ph * Hkv + g) * (uint32_t)(kTileU4 * 16) : 0u;
    }
    const int tok0 = (blk_lo + 2 * st) * kBlock;
    const bool full = ok2 == 3u && tok0 + 31 < L && tok0 + 31 <= qpos_lo &&
                      (a.window <= 0 || qpos_hi - tok0 < a.window);
    const bool tail = !(ok2 == 3u && tok0 + 2 * kBlock <= L);
    const int slot = st & (NB - 1);
    okbits = (okbits & ~(3u << (2 * slot))) | (ok2 << (2 * slot));
    fullbits = (fullbits & ~(1u << slot)) | ((uint32_t)full << slot);
    tailbits = (tailbits & ~(1u << slot)) | ((uint32_t)tail << slot);
    cdst = smem + slot * kStageU4;
  };
  // With per-block descriptors (pools over 4 GiB) a copy's 1 KiB run offset
  // goes to the scalar offset, so that all of a wave's copies share one
  // lane-offset register for K and one for V: the descriptors take registers
  // the loop would otherwise spill for.
  const int k_lane = k_off * 16, v_lane = v_off * 16;
  auto copy = [&](int j) {
    if (j < KD / kWaves) {
      const int pr = 2 * j + (wave >> 1);
      u32x4* dst = cdst + pr * 2 * kWave + (wave & 1) * kWave;
      if constexpr (FLAT)
        copy_to_lds(rkp, (64 * pr + k_off) * 16, csoff, dst);
      else
        copy_to_lds((wave & 1) ? crk1 : crk0, k_lane, pr * 1024, dst);
    } else {
      const int x = 2 * (j - KD / kWaves) + (wave >> 1);
      u32x4* dst = cdst + (KD + 2 * x + (wave & 1)) * kWave;
      if constexpr (FLAT)
        copy_to_lds(rvp, (64 * x + v_off) * 16, csoff, dst);
      else
        copy_to_lds((wave & 1) ? crv1 : crv0, v_lane, x * 1024, dst);
    }
  };

  auto k_run = [](int s) { return (s >> 1) * 2 * kWave + (s & 1) * 32; };
  auto stage_tok0 = [&](int st) { return (blk_lo + 2 * st) * kBlock; };
  auto stage_ok = [&](int st) { return (okbits >> (2 * (st & (NB - 1)))) & 3u; };
  auto stage_full = [&](int st) { return (fullbits >> (st & (NB - 1))) & 1u; };
  auto stage_tail = [&](int st) { return (tailbits >> (st & (NB - 1))) & 1u; };

  f32x16 o[XT];
#pragma unroll
  for (int x = 0; x < XT; ++x) o[x] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  constexpr float kLazy = 8.0f;  // rescale only when the max grows by 2^8

  // prologue: the copies of intervals 0 .. kAheadIv - 1
  for (int iv = 0; iv < kAheadIv; ++iv) {
    const int st = 2 * iv + half;
    if (st < nstage) {
      prepare(st);
#pragma unroll
      for (int j = 0; j < kDma; ++j) copy(j);
    }
  }

  for (int iv = 0; iv < n_iv; ++iv) {
    // this wave's copies of interval iv have landed (those of later intervals
    // may still be in flight, unless there are none: the last intervals)
    if constexpr (kAheadIv > 1) {
      if (2 * (iv + kAheadIv - 1) + half < nstage)
        wait_vmem<(kAheadIv - 1) * kDma>();
      else
        wait_vmem<0>();
    } else {
      wait_vmem<0>();
    }
    lds_barrier();  // ... and every other wave's; interval iv - 1 is done
    const int st = 2 * iv + half;
    const int st_copy = st + 2 * kAheadIv;
    const bool do_copy = st_copy < nstage;
    if (do_copy) prepare(st_copy);
    if (!(wave_live && st < nstage)) {
      if (do_copy) {
#pragma unroll
        for (int j = 0; j < kDma; ++j) copy(j);
      }
      continue;
    }
    const int slot = st & (NB - 1);

    // S^T = K Q^T, with this interval's copies issued in its shadow (two
    // instances of the loop, so that no branch sits between the products)
    const u32x4* kb = smem + slot * kStageU4 + k_rd;
    f32x16 acc = {};
    auto qk = [&](auto with_copies) {
      u32x4 kf[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) kf[i] = kb[k_run(i)];
#pragma unroll
      for (int i = 0; i < KD; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        acc = mma32_bf16(kf[i % kAhead], qf[i], acc);
        if (i + kAhead < KD) kf[i % kAhead] = kb[k_run(i + kAhead)];
        if constexpr (decltype(with_copies)::value) {
          if ((i & 1) == 0) copy(i >> 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    if (do_copy)
      qk(std::true_type{});
    else
      qk(std::false_type{});

    // keys past the context (or of an unreadable block): their V entries are
    // cleared in LDS before the products read them (every wave computing this
    // stage writes the same values)
    if (stage_tail(st)) {
      const int tok0 = stage_tok0(st);
      const uint32_t okk = stage_ok(st);
      u32x4* vr = smem + slot * kStageU4 + KD * kWave;
      for (int c = lane; c < 2 * XT * kWave; c += kWave) {
        const int q = (c >> 6) & 1, kgc = (c >> 5) & 1;
        const int nv = ((okk >> q) & 1u) ? L - (tok0 + 16 * q) - 8 * kgc : 0;
        if (nv >= 8) continue;
        const u32x4 m = {(0 < nv ? 0x0000FFFFu : 0u) | (1 < nv ? 0xFFFF0000u : 0u),
                         (2 < nv ? 0x0000FFFFu : 0u) | (3 < nv ? 0xFFFF0000u : 0u),
                         (4 < nv ? 0x0000FFFFu : 0u) | (5 < nv ? 0xFFFF0000u : 0u),
                         (6 < nv ? 0x0000FFFFu : 0u) | (7 < nv ? 0xFFFF0000u : 0u)};
        vr[c] = vr[c] & m;
      }
      wait_lds();
    }

    mma_result_fence();
    if (!stage_full(st)) {
      const int tok0 = stage_tok0(st);
      const uint32_t okk = stage_ok(st);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tk = tok0 + 16 * (v >> 3) + 8 * kg + (v & 7);
        const bool vis = ((okk >> (v >> 3)) & 1u) & rvalid & (tk < L) & (tk <= qpos) &
                         ((a.window <= 0) | (qpos - tk < a.window));
        acc[v] = vis ? acc[v] : kNegInf;
      }
    }

    // softmax of the stage: row max (base-2 logits), lazy rescale, then
    // probabilities as bf16 pairs and their row sum
    float mx = kNegInf;
    if constexpr (SC) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float y = softcap_log2(acc[v] * xf.scale, xf.cap, xf.inv_cap);
        acc[v] = acc[v] == kNegInf ? kNegInf : y;
        mx = fmaxf(mx, acc[v]);
      }
      mx = half_max(mx);
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, acc[v]);
      mx = half_max(mx) * pos_scale_log2;
    }
    if (__any(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int x = 0; x < XT; ++x) o[x] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    uint32_t pw[8];
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      float p0, p1;
      if constexpr (SC) {
        p0 = fast_exp2(acc[v] - m_use);
        p1 = fast_exp2(acc[v + 1] - m_use);
      } else {
        p0 = fast_exp2(fmaf(acc[v], pos_scale_log2, -m_use));
        p1 = fast_exp2(fmaf(acc[v + 1], pos_scale_log2, -m_use));
      }
      pw[v >> 1] = pack_bf16x2_hw(p0, p1);
      l_run += p0 + p1;
    }
    const u32x4 pb[2] = {u32x4{pw[0], pw[1], pw[2], pw[3]}, u32x4{pw[4], pw[5], pw[6], pw[7]}};

    // O^T += V^T P^T
    const u32x4* vb = smem + slot * kStageU4 + KD * kWave + lane;
    {
      constexpr int NU = 2 * XT;
      u32x4 vf[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) vf[u] = vb[(2 * (u % XT) + u / XT) * kWave];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        const int x = u % XT, q = u / XT;
        o[x] = mma32_bf16(vf[u % kAhead], pb[q], o[x]);
        if (u + kAhead < NU) vf[u % kAhead] = vb[(2 * ((u + kAhead) % XT) + (u + kAhead) / XT) * kWave];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmem<0>();  // no copy in flight: the ring is reused below
  mma_result_fence();
  lds_barrier();   // every wave is done with the ring

  // merge the pair: each wave finalises half of the output tiles, taking the
  // other half's partial (and its max and sum) through LDS
  constexpr int XH = XT / 2;
  constexpr int kXchg = XH * 16 * kWave + 2 * kWave;  // floats per wave
  const float l_tot = half_sum(l_run);
  float* xw = reinterpret_cast<float*>(smem) + w * kXchg;
  if (wave_live) {
#pragma unroll
    for (int x2 = 0; x2 < XH; ++x2) {
      // the tiles the partner finalises (constant register indices, a select)
      f32x16 t;
#pragma unroll
      for (int e = 0; e < 16; ++e) t[e] = half ? o[x2][e] : o[XH + x2][e];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<f32x4*>(xw + ((x2 * 4 + c) * kWave + lane) * 4) =
            f32x4{t[4 * c], t[4 * c + 1], t[4 * c + 2], t[4 * c + 3]};
    }
    *reinterpret_cast<f32x2*>(xw + XH * 16 * kWave + 2 * lane) = f32x2{m_run, l_tot};
  }
  lds_barrier();
#ifdef PKV_TIMELINE
  if (threadIdx.x == 0 && a.timeline != nullptr && blk < kTimelineWgs) {
    unsigned long long* tl = a.timeline + (size_t)blk * kTimelineStamps;
    tl[0] = tl_cyc0;
    tl[1] = __builtin_amdgcn_s_memtime();
    tl[2] = tl_rt0;
    tl[3] = __builtin_amdgcn_s_memrealtime();
    tl[4] = (unsigned long long)nstage;
    tl[5] = (unsigned long long)tile;
  }
#endif
  if (!wave_live) return;
  // the partner's exchange area: its partial of this wave's half, read whole
  // into registers first (after that nobody reads this area again, and it
  // stages this wave's output rows below)
  float* xp = reinterpret_cast<float*>(smem) + (w ^ 4) * kXchg;
  const f32x2 ml = *reinterpret_cast<const f32x2*>(xp + XH * 16 * kWave + 2 * lane);
  f32x4 pv[XH * 4];
#pragma unroll
  for (int q = 0; q < XH * 4; ++q) pv[q] = *reinterpret_cast<const f32x4*>(xp + (q * kWave + lane) * 4);
  const float M = fmaxf(m_run, ml[0]);
  const float mu = M == kNegInf ? 0.f : M;
  const float a_self = fast_exp2(m_run - mu), a_part = fast_exp2(ml[0] - mu);
  const float Lt = l_tot * a_self + ml[1] * a_part;
  if (half == 0 && a.lse != nullptr && kg == 0 && rvalid)
    a.lse[(size_t)(r0 + pos) * Hq + head] = Lt > 0.f ? (M + fast_log2(Lt)) * kLn2 : kNegInf;
  const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;
  const float cs = a_self * inv, cp = a_part * inv;
  // The rows leave through LDS so that a wave writes whole 128-byte lines (a
  // row's half is D bytes: D / 16 lanes of 16 bytes) with streaming stores,
  // which go to memory as the workgroup finishes instead of waiting in L2 as
  // partial lines.  Staged row-halves are padded by 16 bytes against bank
  // conflicts.
  constexpr int kRowU32 = D / 4 + 4;
  uint32_t* stage = reinterpret_cast<uint32_t*>(xp);
#pragma unroll
  for (int x2 = 0; x2 < XH; ++x2) {
    f32x16 t;  // this wave's tile (element-wise select: the array stays in registers)
#pragma unroll
    for (int e = 0; e < 16; ++e) t[e] = half ? o[XH + x2][e] : o[x2][e];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const f32x4 v = pv[x2 * 4 + h];
      *reinterpret_cast<u32x2*>(stage + n * kRowU32 + 16 * x2 + 4 * h + 2 * kg) =
          u32x2{pack_bf16x2_hw(t[4 * h] * cs + v[0] * cp, t[4 * h + 1] * cs + v[1] * cp),
                pack_bf16x2_hw(t[4 * h + 2] * cs + v[2] * cp, t[4 * h + 3] * cs + v[3] * cp)};
    }
  }
  wait_lds();
  constexpr int kLanesPerRow = D / 16;  // 16-byte pieces of a row-half
  constexpr int kRowsPerStep = kWave / kLanesPerRow;
  const int col = lane % kLanesPerRow;
#pragma unroll
  for (int r0w = 0; r0w < 32; r0w += kRowsPerStep) {
    const int r = r0w + lane / kLanesPerRow;
    const int rpos = pos_wave + r / G;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * kRowU32 + 4 * col);
    if (rpos < nq) {
      uint16_t* row = reinterpret_cast<uint16_t*>(a.out) + ((size_t)(r0 + rpos) * Hq + g * G + r % G) * D;
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(row + half * (D / 2) + 8 * col));
    }
  }
}

template <int D, int NB, bool SC, bool FLAT>
__global__ __launch_bounds__(2 * kThreads, 1) void prefill_pp_kernel(PrefillArgs a) {
  __shared__ u32x4 smem[kPrefillPPLdsBytes<D, NB> / 16];
  prefill_pp_body<D, NB, SC, FLAT>(a, blockIdx.x, smem);
}

// each pool addressable by one buffer descriptor (32-bit offsets)
template <int D>
bool prefill_flat(const PrefillArgs& a) {
  return (unsigned long long)a.num_blocks * a.num_kv_heads * D * kBlock * 2 <= 0xFFFFFFFFull;
}

template <int D>
void launch_mma32(PrefillArgs a, hipStream_t stream) {
  const bool flat = prefill_flat<D>(a);
  constexpr int T = 2 * kThreads;
  if (a.softcap > 0.f) {
    if (flat)
      prefill_pp_kernel<D, PKV_PREFILL_RING, true, true><<<a.num_items, T, 0, stream>>>(a);
    else
      prefill_pp_kernel<D, PKV_PREFILL_RING, true, false><<<a.num_items, T, 0, stream>>>(a);
  } else {
    if (flat)
      prefill_pp_kernel<D, PKV_PREFILL_RING, false, true><<<a.num_items, T, 0, stream>>>(a);
    else
      prefill_pp_kernel<D, PKV_PREFILL_RING, false, false><<<a.num_items, T, 0, stream>>>(a);
  }
}

template <bool BF16, int D, int RT>
hipError_t launch_p(PrefillArgs a, hipStream_t stream) {
  const int pos_per_item = kWaves * RT * (16 / a.gqa_group);
  // tiles_per_seq was sized by the host for this RT
  if (a.tiles_per_seq * pos_per_item <= 0) return hipErrorInvalidValue;
  prefill_kernel<BF16, D, RT><<<a.num_items, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

#ifndef PKV_ATTN_BODIES_ONLY
// Row tiles per wave of the bf16 (LDS) form, and of the fp32 form.
int prefill_row_tiles(int head_dim, bool bf16) {
  if (bf16) return 2;  // 32 rows per wave
  return head_dim >= 256 ? 1 : 2;
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  if (a.num_items <= 0) return hipSuccess;
  if (bf16) {
    hipError_t e = hipSuccess;
    switch (head_dim) {
      case 64: launch_mma32<64>(a, stream); break;
      case 128: launch_mma32<128>(a, stream); break;
      case 256: launch_mma32<256>(a, stream); break;
      default: e = hipErrorInvalidValue;
    }
    return e != hipSuccess ? e : hipGetLastError();
  } else {
    switch (head_dim) {
      case 64: return launch_p<false, 64, 2>(a, stream);
      case 128: return launch_p<false, 128, 2>(a, stream);
      case 256: return launch_p<false, 256, 1>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

#endif

}  // namespace pkv
