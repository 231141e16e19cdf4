// Batched one-token decode over the block-paged cache, and its split-K form.
//
// Pages: "Inference Server" (project README mirror), section "The engine" --
// paged decode reading K/V through block tables, a split-K decode variant;
// "Inference Server -- Architecture Map", section "How a single request flows
// through the system" -- one batched decode per tick over all active
// sequences.
//
// Work decomposition.  A unit of work is one cache block of one (sequence,
// kv head) "segment": 16 tokens of K and V.  All units are laid out segment
// after segment.
//   * balanced mode (paged_attn_decode): workgroup w takes the contiguous
//     range [w W / N, (w+1) W / N) of the W units, whatever their lengths,
//     so every CU streams the same number of bytes however ragged the batch.
//   * fixed mode (paged_attn_decode_splitk): workgroup (segment, p) takes the
//     blocks of partition p, tokens [p P, (p+1) P).
// A workgroup's range meets one or more segments; the part of its range
// inside one segment is a "piece".  Its four waves share the piece's blocks
// round-robin, each with its own online softmax, and combine through LDS.  A
// piece that is a whole segment writes the output directly; otherwise it
// stores (max, sum, unnormalised output) to the workspace.  A second, small
// kernel then merges the pieces of every split segment by log-sum-exp.  The
// kernel boundary is what makes the partials visible to the merge: a merge
// inside the same launch would need device-scope release/acquire fences, and
// on a multi-XCD part each of those writes back and invalidates an XCD's whole
// L2, which serialises and costs more than the extra launch.
//
// Inner loop per wave: double-buffered block loads (K and V fragments for
// the next block are in flight while the current block is computed), S^T =
// K Q^T on the matrix cores with the GQA group's query heads as the 16
// columns (padded with zero rows), mask by select, online softmax in base 2
// with cross-lane max over the 4 lanes that share a head, then P V on the
// matrix cores.
#include <type_traits>

#include "attn_tile.hpp"
#include "launch.hpp"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;

struct Piece {
  int b, g;       // sequence, kv head
  SeqSpan sp;     // its visible range
  int j0, j1;     // blocks [j0, j1) of the segment's visible blocks
  int slot;       // workspace slot if partial
  long long S;    // flattened index of the segment's first unit (balanced mode)
};

template <bool BF16, int D>
__device__ __forceinline__ void finalize_vec(const DecodeArgs& a, int b, int h_global, int d,
                                             f32x4 O, float L, float M) {
  using T = typename Elem<BF16>::T;
  const int Hq = a.num_kv_heads * a.gqa_group;
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  store4(reinterpret_cast<T*>(a.out) + ((size_t)b * Hq + h_global) * D + d, O * inv);
  if (d == 0 && a.lse != nullptr)
    a.lse[(size_t)b * Hq + h_global] = L > 0.f ? (M + fast_log2(L)) * kLn2 : kNegInf;
}

// Merge the partials listed by `slots` for query head h of segment (b, g)
// and write its output row.  Thread (group, lane) takes the slots k = group,
// group + kGroups, ... for dims 4 lane .. 4 lane + 3; it issues the loads of
// up to kPer slots at once, then folds them into a running (max, sum,
// output); the groups are folded through LDS at the end.
template <bool BF16, int D, typename SlotList>
__device__ void merge_row(const DecodeArgs& a, int b, int g, int h, SlotList slots, float* lds) {
  constexpr int kLanes = D / 4;                 // float4 columns per row
  constexpr int kGroups = kThreads / kLanes;    // slot groups (16, 8 or 4)
  constexpr int kPer = 8;                       // slots in flight per thread
  const int G = a.gqa_group;
  const int col = threadIdx.x % kLanes, grp = threadIdx.x / kLanes;
  float M = kNegInf, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  const int cnt = slots.count();
  for (int k0 = grp; k0 < cnt; k0 += kGroups * kPer) {
    float mk[kPer], lk[kPer];
    f32x4 ov[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int k = k0 + q * kGroups;
      int sl = 0;
      const bool valid = k < cnt && slots.slot(k, sl);
      lk[q] = 0.f;
      mk[q] = kNegInf;
      ov[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (valid) {
        mk[q] = a.part_ml[((size_t)sl * G + h) * 2];
        lk[q] = a.part_ml[((size_t)sl * G + h) * 2 + 1];
        ov[q] = *reinterpret_cast<const f32x4*>(a.part_o + ((size_t)sl * G + h) * D + 4 * col);
      }
    }
    float Mn = M;
#pragma unroll
    for (int q = 0; q < kPer; ++q) Mn = lk[q] > 0.f ? fmaxf(Mn, mk[q]) : Mn;
    if (Mn != kNegInf) {
      const float sa = fast_exp2(M - Mn);  // 0 when M = -inf
      O = O * sa;
      L = L * sa;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const float sb = lk[q] > 0.f ? fast_exp2(mk[q] - Mn) : 0.f;
        O += ov[q] * sb;
        L += lk[q] * sb;
      }
      M = Mn;
    }
  }
  if constexpr (kGroups > 1) {
    f32x4* lo = reinterpret_cast<f32x4*>(lds);          // [kGroups][kLanes]
    float* lml = lds + 4 * kGroups * kLanes;             // [kGroups][2]
    lo[grp * kLanes + col] = O;
    if (col == 0) {
      lml[2 * grp] = M;
      lml[2 * grp + 1] = L;
    }
    __syncthreads();
    if (grp == 0) {
      float Mt = kNegInf;
#pragma unroll
      for (int q = 0; q < kGroups; ++q) Mt = fmaxf(Mt, lml[2 * q]);
      O = f32x4{0.f, 0.f, 0.f, 0.f};
      L = 0.f;
      if (Mt != kNegInf) {
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
          const float sc = fast_exp2(lml[2 * q] - Mt);
          O += lo[q * kLanes + col] * sc;
          L += lml[2 * q + 1] * sc;
        }
      }
      M = Mt;
    }
  }
  if (grp == 0) finalize_vec<BF16, D>(a, b, g * G + h, 4 * col, O, L, M);
}

struct SplitSlots {  // fixed partitions p_lo .. p_hi of one segment
  int base, p_lo, p_hi;
  __device__ int count() const { return p_hi - p_lo + 1; }
  __device__ bool slot(int k, int& s) const {
    s = base + p_lo + k;
    return true;
  }
};

struct BalancedSlots {  // workgroups whose ranges meet [S, E)
  long long W, S, E;
  int N, w_first, w_last;
  __device__ BalancedSlots(long long W_, long long S_, long long E_, int N_)
      : W(W_), S(S_), E(E_), N(N_) {
    w_first = (int)(((S + 1) * N - 1) / W);
    w_last = (int)((E * N - 1) / W);
  }
  __device__ int count() const { return w_last - w_first + 1; }
  __device__ bool slot(int k, int& s) const {
    const int w = w_first + k;
    const long long a0 = (long long)w * W / N, a1 = (long long)(w + 1) * W / N;
    s = a0 < S ? 2 * w + 1 : 2 * w;
    return a0 < a1;  // an empty range wrote nothing
  }
};

// One piece: all four waves of the workgroup.
template <bool BF16, int D>
__device__ void run_piece(const DecodeArgs& a, const LogitXform& xf, const Piece& pc, float* lds) {
  using T = typename Elem<BF16>::T;
  using KV = KVFrag<BF16, D>;
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  // wave index as a uniform (scalar) value: table lookups become scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, j = lane >> 4;
  const int G = a.gqa_group, Hkv = a.num_kv_heads, Hq = G * Hkv;
  const int b = pc.b, g = pc.g;
  const SeqSpan& sp = pc.sp;

  QFrag<BF16, D> qf;
  if (c < G)
    qf.load(reinterpret_cast<const T*>(a.q) + ((size_t)b * Hq + g * G + c) * D, lane);
  else
    qf.zero();

  f32x4 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const int* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq + sp.first_blk;
  const T* kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* vpool = reinterpret_cast<const T*>(a.v_pool);
  constexpr size_t kTile = (size_t)D * kBlock;

  // This wave's blocks: j0 + wave + 4 i, i < nw.  Their table entries are
  // read 64 at a time, one per lane, and picked out with readlane, so the
  // block loop itself touches memory only for K and V.
  const int span = pc.j1 - pc.j0 - wave;
  const int nw = span > 0 ? (span + kWaves - 1) / kWaves : 0;
  int tbl = 0;

  // One K and one V register set.  K of block i + 1 is loaded as soon as the
  // score product of block i has consumed K, V of block i + 1 as soon as the
  // P V product has consumed V: about one block stays in flight per wave with
  // a single buffer, which keeps the wave within 256 registers (two waves per
  // SIMD).  An out-of-range table entry loads block 0 and is masked out, so
  // loads are never conditional inside the loop (exact compiler wait counts);
  // the last block, which prefetches nothing, is peeled off.
  auto tile = [&](int i, bool& ok) -> size_t {
    const int phys = __builtin_amdgcn_readlane(tbl, i & 63);
    ok = (unsigned)phys < (unsigned)a.num_blocks;
    return ((size_t)(ok ? phys : 0) * Hkv + g) * kTile;
  };

  KV buf;
  bool ok = false;
  size_t off = 0;
  // rows whose running max rose by more than this (log2 units) since the last
  // rescale trigger one; below it, weights up to 2^8 are accumulated as is
  constexpr float kLazy = 8.0f;

  auto body = [&](int i, auto prefetch) {
    constexpr bool PF = decltype(prefetch)::value;
    const int tok0 = (sp.first_blk + pc.j0 + wave + kWaves * i) * kBlock;
    const f32x4 sc = qk_tile<D>(buf, qf);
    bool ok_next = false;
    size_t off_next = 0;
    if constexpr (PF) {
      off_next = tile(i + 1, ok_next);
      buf.load_k(kpool + off_next, lane);
    }
    float s2[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tok0 + 4 * j + r;
      const bool vis = ok & (t >= sp.vis_lo) & (t < sp.L);
      s2[r] = vis ? xf(sc[r]) : kNegInf;
    }
    float mx = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__any(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
      l_run *= alpha;
      // O rows are heads 4j + r: fetch their factors from lanes 4j + r
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * j + r);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        o[t].x *= ar[0];
        o[t].y *= ar[1];
        o[t].z *= ar[2];
        o[t].w *= ar[3];
      }
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s2[r] - m_use);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    if (!ok)
      buf.zero_v();
    else if (tok0 + kBlock > sp.L)
      buf.mask_v_tail(sp.L - tok0, lane);
    pv_tile<D>(o, p, buf);
    if constexpr (PF) {
      mma_result_fence();  // the products have read V before it is reloaded
      buf.load_v(vpool + off_next, lane);
      ok = ok_next;
    }
  };

  for (int base = 0; base < nw; base += 64) {
    const int cnt = min(64, nw - base);
    tbl = lane < cnt ? bt[pc.j0 + wave + kWaves * (base + lane)] : 0;
    if constexpr (kPrefetch<BF16, D>) {
      off = tile(0, ok);
      buf.load(kpool + off, vpool + off, lane);
      int i = 0;
      for (; i + 1 < cnt; ++i) body(base + i, std::true_type{});
      body(base + i, std::false_type{});
    } else {  // fragments too large to refill early: load, then compute
      for (int i = 0; i < cnt; ++i) {
        off = tile(base + i, ok);
        buf.load(kpool + off, vpool + off, lane);
        body(base + i, std::false_type{});
      }
    }
  }

  // ---- combine the four waves through LDS ----
  mma_result_fence();
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float* lo = lds;                      // [4][G][D]
  float* lml = lds + kWaves * G * D;    // [4][G][2]
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * j + r;
      if (h < G) lo[((size_t)wave * G + h) * D + t * 16 + c] = o[t][r];
    }
  }
  if (j == 0 && c < G) {
    lml[(wave * G + c) * 2] = m_run;
    lml[(wave * G + c) * 2 + 1] = l_tot;
  }
  __syncthreads();

  const bool whole = (pc.j0 == 0 && pc.j1 == sp.nb);
  const int nvec = G * D / 4;
  for (int e = threadIdx.x; e < nvec; e += kThreads) {
    const int h = (e * 4) / D, d = (e * 4) % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lml[(w * G + h) * 2]);
    float L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float s = fast_exp2(lml[(w * G + h) * 2] - M);
        L += lml[(w * G + h) * 2 + 1] * s;
        O += *reinterpret_cast<const f32x4*>(lo + ((size_t)w * G + h) * D + d) * s;
      }
    }
    if (whole) {
      finalize_vec<BF16, D>(a, b, g * G + h, d, O, L, M);
    } else {
      *reinterpret_cast<f32x4*>(a.part_o + ((size_t)pc.slot * G + h) * D + d) = O;
      if (d == 0) {
        a.part_ml[((size_t)pc.slot * G + h) * 2] = M;
        a.part_ml[((size_t)pc.slot * G + h) * 2 + 1] = L;
      }
    }
  }

  __syncthreads();  // LDS is reused by the next piece
}

// Blocks in flight per workgroup in the split-D form (ring of buffers).
#ifndef PKV_DECODE_SD_NBUF
#define PKV_DECODE_SD_NBUF 4
#endif

// One piece, split-D form (bf16): all four waves walk the same blocks; wave
// w owns head dims [w D/4, (w+1) D/4): its slices of q, K, V and of the
// output accumulators.  Score partials are summed through LDS (double-
// buffered, one barrier per block, every wave adding the four partials in
// the same order so that all waves hold identical softmax weights), then
// each wave runs P V on its V slice.  Per-wave state is a quarter of the
// per-wave-block form, so more waves fit per SIMD.
template <int D>
__device__ void run_piece_sd(const DecodeArgs& a, const LogitXform& xf, const Piece& pc,
                             f32x4* xs) {
  constexpr int KW = D / 32 / kWaves;  // score k-steps per wave
  constexpr int NW = D / 16 / kWaves;  // P V column tiles per wave
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, j = lane >> 4;
  const int G = a.gqa_group, Hkv = a.num_kv_heads, Hq = G * Hkv;
  const int b = pc.b, g = pc.g;
  const SeqSpan& sp = pc.sp;

  u32x4 qf[KW];
  const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * Hq + g * G + c) * D;
#pragma unroll
  for (int s = 0; s < KW; ++s)
    qf[s] = c < G ? *reinterpret_cast<const u32x4*>(qrow + (4 * (wave * KW + s) + j) * 8)
                  : u32x4{0, 0, 0, 0};

  f32x4 o[NW];
#pragma unroll
  for (int t = 0; t < NW; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  constexpr float kLazy = 8.0f;

  struct Slice {
    u32x4 k[KW];
    u32x2 v[NW];
  };
  const int* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq + sp.first_blk + pc.j0;
  const uint16_t* kpool = reinterpret_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vpool = reinterpret_cast<const uint16_t*>(a.v_pool);
  constexpr size_t kTile = (size_t)D * kBlock;
  int tbl = 0;

  auto fetch = [&](Slice& buf, int i) -> bool {
    const int phys = __builtin_amdgcn_readlane(tbl, i & 63);
    const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
    const size_t off = ((size_t)(ok ? phys : 0) * Hkv + g) * kTile;
    const uint16_t* kt = kpool + off + (size_t)wave * KW * kWave * 8;
    const uint16_t* vt = vpool + off + (size_t)wave * NW * 16 * kBlock;
#pragma unroll
    for (int s = 0; s < KW; ++s) buf.k[s] = *reinterpret_cast<const u32x4*>(kt + (s * kWave + lane) * 8);
#pragma unroll
    for (int t = 0; t < NW; ++t)
      buf.v[t] = *reinterpret_cast<const u32x2*>(vt + (t * 16 + c) * kBlock + 4 * j);
    return ok;
  };

  auto step = [&](Slice& buf, bool ok, int i) {
    const int tok0 = (sp.first_blk + pc.j0 + i) * kBlock;
    f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KW; ++s) part = mma_bf16_k32(buf.k[s], qf[s], part);
    mma_result_fence();
    f32x4* x = xs + (i & 1) * kWaves * kWave;
    x[wave * kWave + lane] = part;
    __syncthreads();
    const f32x4 sc = ((x[lane] + x[kWave + lane]) + x[2 * kWave + lane]) + x[3 * kWave + lane];
    float s2[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tok0 + 4 * j + r;
      const bool vis = ok & (t >= sp.vis_lo) & (t < sp.L);
      s2[r] = vis ? xf(sc[r]) : kNegInf;
    }
    float mx = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__any(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
      l_run *= alpha;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * j + r);
#pragma unroll
      for (int t = 0; t < NW; ++t) {
        o[t].x *= ar[0];
        o[t].y *= ar[1];
        o[t].z *= ar[2];
        o[t].w *= ar[3];
      }
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s2[r] - m_use);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    if (!ok) {
#pragma unroll
      for (int t = 0; t < NW; ++t) buf.v[t] = u32x2{0, 0};
    } else if (tok0 + kBlock > sp.L) {
      const int nv = sp.L - tok0, t0 = 4 * j;
      const uint32_t lo = (t0 + 0 < nv ? 0x0000FFFFu : 0u) | (t0 + 1 < nv ? 0xFFFF0000u : 0u);
      const uint32_t hi = (t0 + 2 < nv ? 0x0000FFFFu : 0u) | (t0 + 3 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int t = 0; t < NW; ++t) buf.v[t] = u32x2{buf.v[t].x & lo, buf.v[t].y & hi};
    }
    const u32x2 pa = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
#pragma unroll
    for (int t = 0; t < NW; ++t) o[t] = mma_bf16_k16(pa, buf.v[t], o[t]);
  };

  const int nblk = pc.j1 - pc.j0;
  for (int base = 0; base < nblk; base += 64) {
    const int cnt = min(64, nblk - base);
    tbl = lane < cnt ? bt[base + lane] : 0;
    walk_ring<PKV_DECODE_SD_NBUF, Slice>(
        cnt, fetch, [&](Slice& buf, bool ok, int i) { step(buf, ok, base + i); });
  }
  mma_result_fence();

  // row totals and this wave's slice of the output (or of the partial)
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const bool whole = (pc.j0 == 0 && pc.j1 == sp.nb);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * j + r;
    const float lh = __shfl(l_tot, h);
    if (h >= G) continue;
    const int d0 = 16 * wave * NW + c;
    if (whole) {
      const float inv = lh > 0.f ? 1.0f / lh : 0.f;
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + ((size_t)b * Hq + g * G + h) * D + d0;
#pragma unroll
      for (int t = 0; t < NW; ++t) store1(dst + 16 * t, o[t][r] * inv);
    } else {
      float* dst = a.part_o + ((size_t)pc.slot * G + h) * D + d0;
#pragma unroll
      for (int t = 0; t < NW; ++t) dst[16 * t] = o[t][r];
    }
  }
  if (wave == 0 && j == 0 && c < G) {
    if (whole) {
      if (a.lse != nullptr)
        a.lse[(size_t)b * Hq + g * G + c] =
            l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    } else {
      a.part_ml[((size_t)pc.slot * G + c) * 2] = m_run;
      a.part_ml[((size_t)pc.slot * G + c) * 2 + 1] = l_tot;
    }
  }
  __syncthreads();  // the exchange buffer is reused by the next piece
}

// Output of a sequence with nothing to attend to: 0, lse = -inf.
template <bool BF16, int D>
__device__ void write_empty(const DecodeArgs& a, int b, int h_lo, int h_hi) {
  using T = typename Elem<BF16>::T;
  const int Hq = a.num_kv_heads * a.gqa_group;
  const int n = (h_hi - h_lo) * D / 4;
  for (int e = threadIdx.x; e < n; e += kThreads) {
    const int h = h_lo + (e * 4) / D, d = (e * 4) % D;
    store4(reinterpret_cast<T*>(a.out) + ((size_t)b * Hq + h) * D + d, f32x4{0.f, 0.f, 0.f, 0.f});
    if (d == 0 && a.lse != nullptr) a.lse[(size_t)b * Hq + h] = kNegInf;
  }
}

template <bool BF16, int D, bool FIXED, bool SD>
__global__ __launch_bounds__(kThreads, SD ? 2 : 1) void decode_kernel(DecodeArgs a) {
  extern __shared__ float lds[];
  auto run_one = [&](const LogitXform& xf, const Piece& pc) {
    if constexpr (SD)
      run_piece_sd<D>(a, xf, pc, reinterpret_cast<f32x4*>(lds));
    else
      run_piece<BF16, D>(a, xf, pc, lds);
  };
  const LogitXform xf = make_xform(a.scale, a.softcap);
  const int Hkv = a.num_kv_heads, G = a.gqa_group;

  if constexpr (FIXED) {
    const int NP = a.num_partitions, PB = a.part_blocks;
    const int seg = blockIdx.x / NP, p = blockIdx.x % NP;
    const int b = seg / Hkv, g = seg % Hkv;
    Piece pc;
    pc.b = b;
    pc.g = g;
    pc.sp = seq_span(a.context_lens[b], a.window, a.max_context_len);
    if (pc.sp.nb == 0) {
      if (p == 0) write_empty<BF16, D>(a, b, g * G, (g + 1) * G);
      return;
    }
    const int last_blk = pc.sp.first_blk + pc.sp.nb - 1;
    const int lo = max(p * PB, pc.sp.first_blk), hi = min((p + 1) * PB - 1, last_blk);
    if (lo > hi) return;  // partition outside the visible range
    pc.j0 = lo - pc.sp.first_blk;
    pc.j1 = hi - pc.sp.first_blk + 1;
    pc.slot = seg * NP + p;
    pc.S = 0;
    run_one(xf, pc);
  } else {
    const int N = a.num_workers, w = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int B = a.num_seqs;

    // sequences with no visible token
    for (int b = w; b < B; b += N) {
      if (seq_span(a.context_lens[b], a.window, a.max_context_len).nb == 0)
        write_empty<BF16, D>(a, b, 0, Hkv * G);
    }

    // total units W (every wave computes the same value)
    long long W = 0;
    for (int base = 0; base < B; base += kWave) {
      const int b = base + lane;
      const int nb = b < B ? seq_span(a.context_lens[b], a.window, a.max_context_len).nb : 0;
      W += wave_sum_i64(nb);
    }
    W *= Hkv;
    const long long a0 = (long long)w * W / N, a1 = (long long)(w + 1) * W / N;
    if (a0 >= a1) return;

    // segment holding unit a0: first sequence whose inclusive prefix exceeds a0
    long long run = 0, seg_base = 0;
    int b0 = 0;
    for (int base = 0; base < B; base += kWave) {
      const int b = base + lane;
      const long long nbh =
          b < B ? (long long)seq_span(a.context_lens[b], a.window, a.max_context_len).nb * Hkv
                : 0;
      const long long incl = wave_incl_scan_i64(nbh, lane);
      const unsigned long long hit = __ballot(run + incl > a0);
      if (hit) {
        const int l0 = __ffsll(hit) - 1;
        b0 = base + l0;
        seg_base = run + __shfl(incl - nbh, l0);
        break;
      }
      run += __shfl(incl, kWave - 1);
    }

    Piece pc;
    pc.b = b0;
    pc.sp = seq_span(a.context_lens[b0], a.window, a.max_context_len);
    pc.g = (int)((a0 - seg_base) / pc.sp.nb);
    pc.S = seg_base + (long long)pc.g * pc.sp.nb;
    long long pos = a0;
    bool first = true;
    while (pos < a1) {
      const long long E = pc.S + pc.sp.nb;
      pc.j0 = (int)(pos - pc.S);
      pc.j1 = (int)(min(a1, E) - pc.S);
      pc.slot = first ? 2 * w : 2 * w + 1;
      run_one(xf, pc);
      first = false;
      pos = E;
      pc.S = E;
      if (pos >= a1) break;
      if (++pc.g == Hkv) {
        pc.g = 0;
        do {
          if (++pc.b >= B) return;
          pc.sp = seq_span(a.context_lens[pc.b], a.window, a.max_context_len);
        } while (pc.sp.nb == 0);
      }
    }
  }
}

// Merge the pieces of segment (b, g) if it was split; one workgroup per
// (segment, query head).  Runs after decode_kernel on the same stream.
template <bool BF16, int D, bool FIXED>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeArgs a) {
  __shared__ float lds[4 * kThreads + 2 * 16];  // kGroups <= 16
  const int Hkv = a.num_kv_heads, G = a.gqa_group;
  const int h = blockIdx.x % G, seg = blockIdx.x / G;
  const int b = seg / Hkv, g = seg % Hkv;
  const SeqSpan sp = seq_span(a.context_lens[b], a.window, a.max_context_len);
  if (sp.nb == 0) return;  // written as empty by decode_kernel
  if constexpr (FIXED) {
    const int NP = a.num_partitions, PB = a.part_blocks;
    const int p_lo = sp.first_blk / PB, p_hi = (sp.first_blk + sp.nb - 1) / PB;
    if (p_lo == p_hi) return;  // one partition: written directly
    merge_row<BF16, D>(a, b, g, h, SplitSlots{seg * NP, p_lo, p_hi}, lds);
  } else {
    // S: units before this segment; W: all units (every wave computes both)
    const int lane = threadIdx.x & 63;
    long long before = 0, W = 0;
    for (int base = 0; base < a.num_seqs; base += kWave) {
      const int bb = base + lane;
      const long long nb =
          bb < a.num_seqs ? seq_span(a.context_lens[bb], a.window, a.max_context_len).nb : 0;
      W += wave_sum_i64(nb);
      before += wave_sum_i64(bb < b ? nb : 0);
    }
    W *= Hkv;
    const long long S = before * Hkv + (long long)g * sp.nb, E = S + sp.nb;
    const int N = a.num_workers;
    const int w_first = (int)(((S + 1) * N - 1) / W), w_last = (int)((E * N - 1) / W);
    if (w_first == w_last) return;  // inside one workgroup's range: written directly
    merge_row<BF16, D>(a, b, g, h, BalancedSlots{W, S, E, N}, lds);
  }
}

// The combine buffer holds the four waves' partial outputs: up to 66 KiB for
// a group of 16 at head_dim 256, above the default 64 KiB dynamic-LDS limit.
template <typename K>
hipError_t allow_lds(K kernel, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

// Balanced-split grid: workgroups per CU for each kernel form, and a floor on
// the blocks a workgroup gets (tiny batches use fewer workgroups).
#ifndef PKV_DECODE_WGS_PER_CU
#define PKV_DECODE_WGS_PER_CU 1
#endif
#ifndef PKV_DECODE_SD_WGS_PER_CU
#define PKV_DECODE_SD_WGS_PER_CU 2
#endif
#ifndef PKV_DECODE_MIN_BLOCKS_PER_WG
#define PKV_DECODE_MIN_BLOCKS_PER_WG 8
#endif
// smallest head_dim that uses the split-D form (bf16)
#ifndef PKV_DECODE_SD_MIN_D
#define PKV_DECODE_SD_MIN_D 256
#endif

template <bool BF16, int D>
hipError_t launch_d(DecodeArgs a, hipStream_t stream) {
  constexpr bool SD = BF16 && D >= PKV_DECODE_SD_MIN_D;
  if (a.part_blocks == 0) {
    long long n = (a.units_bound + PKV_DECODE_MIN_BLOCKS_PER_WG - 1) / PKV_DECODE_MIN_BLOCKS_PER_WG;
    const long long cap = (long long)a.cu_count * (SD ? PKV_DECODE_SD_WGS_PER_CU : PKV_DECODE_WGS_PER_CU);
    n = min(n, min(cap, (long long)kMaxWorkers));
    a.num_workers = (int32_t)max(n, 1LL);
  }
  const size_t lds = SD ? (size_t)2 * kWaves * kWave * sizeof(f32x4)
                        : (size_t)kWaves * a.gqa_group * (D + 2) * sizeof(float);
  const int rows = a.num_seqs * a.num_kv_heads * a.gqa_group;  // merge: one per (segment, head)
  hipError_t e;
  if (a.part_blocks > 0) {
    if ((e = allow_lds(decode_kernel<BF16, D, true, SD>, lds)) != hipSuccess) return e;
    decode_kernel<BF16, D, true, SD><<<a.num_workers, kThreads, lds, stream>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    merge_kernel<BF16, D, true><<<rows, kThreads, 0, stream>>>(a);
  } else {
    if ((e = allow_lds(decode_kernel<BF16, D, false, SD>, lds)) != hipSuccess) return e;
    decode_kernel<BF16, D, false, SD><<<a.num_workers, kThreads, lds, stream>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    merge_kernel<BF16, D, false><<<rows, kThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dt(const DecodeArgs& a, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<BF16, 64>(a, stream);
    case 128: return launch_d<BF16, 128>(a, stream);
    case 256: return launch_d<BF16, 256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  if (a.num_seqs <= 0) return hipSuccess;
  return bf16 ? launch_dt<true>(a, head_dim, stream) : launch_dt<false>(a, head_dim, stream);
}

}  // namespace pkv
