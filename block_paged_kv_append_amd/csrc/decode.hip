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
// stores (max, sum, unnormalised output) to the workspace and counts itself
// in on the segment's counter, and the workgroup that counts the last piece
// merges them all by log-sum-exp in the same launch.  The partials pass
// between workgroups through device-scope stores and loads, which need no
// cache writeback or invalidation on a multi-XCD part.
//
// Fused append (paged_attn_decode_append): the wave that computes a
// segment's last block takes the newest token's K and V rows from the
// caller's arrays and also writes them to the pool, so one launch does the
// tick's append and its decode.
//
// Inner loop per wave (bf16): S^T = K Q^T on the matrix cores with the GQA
// group's query heads as the 16 columns (zero past the group), mask by
// select, online softmax in base 2 with the row reductions across the four
// lanes that share a head, then O^T += V^T P^T on the matrix cores.  bf16
// blocks stream through per-wave LDS rings filled by direct buffer-to-LDS
// copies; fp32 blocks through registers.
#include <algorithm>
#include <type_traits>

#include "attn_tile.hpp"
#include "launch.hpp"
#include "slots.hpp"

namespace pkv {
namespace {


// Partial results pass between workgroups (possibly on different XCDs, whose
// L2 caches are not coherent with each other) only through device-scope
// accesses: stores written through to the device coherence point and loads
// served from it.  A workgroup completes its partial stores (vmcnt(0))
// before it counts its piece in with an atomic add; the workgroup that
// counts the segment's last piece then reads every partial with device-scope
// loads.  No cache writeback or invalidation is needed (a release/acquire
// fence pair would write back and invalidate a whole L2 per piece).
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-scope stores of 16 and 8 bytes through a buffer resource over a
// region uniform in the workgroup: write-through (sc1) stores, the
// instruction a relaxed agent-scope atomic store of one float compiles to,
// one instruction instead of four.  The merge reads partials the same way,
// 16 bytes per load through a resource over the whole partials region (when
// it spans less than 2 GiB; else per float).
constexpr int kDeviceScope = 16;  // cache policy: sc1
// Cache policy of the K/V copies into the rings: nontemporal.  A decode reads
// every cache block once per launch, so streaming reads keep the blocks from
// displacing anything in the caches (tick 36.0 -> 32.3 us, long-context
// split-K 99.6 -> 88.2 us against the default policy).
constexpr int kStreamLoad = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t region(void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000u);
}
__device__ __forceinline__ void store_dev4(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, kDeviceScope);
}
__device__ __forceinline__ void store_dev2(__amdgpu_buffer_rsrc_t r, int byte_off, float x, float y) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(x), __float_as_uint(y)}, r, byte_off, 0,
                                        kDeviceScope);
}
__device__ __forceinline__ f32x4 load_dev4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kDeviceScope));
}

// Timeline build (PKV_TIMELINE): a workgroup's phases as s_memrealtime
// stamps, written by one lane to a.timeline[blockIdx.x][k]:
//   0 entry, 1 set-up done, 2 first piece's first copies issued (wave 0),
//   3 its first block landed (wave 0), 4 + w last piece's block loop done
//   (wave w), 8 its waves combined, 9 its count-in done, 10 its merge done,
//   11 exit; 12 first piece entered, 13 its copies about to be issued;
//   14 second piece entered, 15 its first copies issued; 16 first piece:
//   its table slice and query fragments have landed (the timeline build
//   waits for them there, before the first copy); last piece: 17 all waves
//   at the combine, 18 their partial outputs in LDS, 19 its partial stores
//   done (count-in), 20 merge: partials loaded.
#ifdef PKV_TIMELINE
__device__ __forceinline__ void tl_put(const DecodeArgs& a, int k, unsigned long long v) {
  if (a.timeline != nullptr && blockIdx.x < (unsigned)kTimelineWgs)
    a.timeline[(size_t)blockIdx.x * kTimelineStamps + k] = v;
}
#define PKV_TL(a, k) \
  do { if (threadIdx.x == 0) tl_put(a, k, __builtin_amdgcn_s_memrealtime()); } while (0)
#define PKV_TL_WAVE(a, k) \
  do { if ((threadIdx.x & 63) == 0) tl_put(a, (k) + (int)(threadIdx.x >> 6), __builtin_amdgcn_s_memrealtime()); } while (0)
#define PKV_TL_VAL(a, k, v) \
  do { if (threadIdx.x == 0) tl_put(a, k, (unsigned long long)(v)); } while (0)
#else
#define PKV_TL(a, k) ((void)0)
#define PKV_TL_WAVE(a, k) ((void)0)
#define PKV_TL_VAL(a, k, v) ((void)0)
#endif

struct Piece {
  int b, g;       // sequence, kv head
  SeqSpan sp;     // its visible range
  int j0, j1;     // blocks [j0, j1) of the segment's visible blocks
  int slot;       // workspace slot if partial
  long long S;    // flattened index of the segment's first unit (balanced mode)
  int ord = 0;    // pieces of this workgroup before it (timeline build)
};

// Fused append (paged_attn_decode_append).  Sequence b's newest token sits
// at position L - 1, in the segment's last visible block; its K and V rows
// come from k_new / v_new [b, g] rather than from the pool.  The wave whose
// blocks include that last block substitutes the rows into its block
// fragments (lanes hold them in the fragments' own layout, loaded when the
// piece starts) and writes them to the pool slot; nothing else in the launch
// reads that block of this kv head, so no ordering with other waves is
// needed.  ESZ is the element size in bytes, E = 16 / ESZ elements per lane
// chunk:
//   K: lane (c, j) holds dims E (4 s + j) .. + E - 1 for every step s
//      (what a lane serving token c reads of a block's K tile)
//   V: lane (c, j) holds dim 16 x + c for every output tile x
template <int ESZ, int D>
struct NewToken {
  static constexpr int E = 16 / ESZ;
  static constexpr int KS = D / (4 * E);      // 16-byte K chunks per lane
  static constexpr int XT = D / 16;           // V elements per lane
  static constexpr int VW = (XT * ESZ) / 4;   // ... in 32-bit words
  u32x4 k[KS];
  uint32_t v[VW];
  bool own = false;  // uniform: this wave computes the segment's last block
  int tn = 0;        // the token's offset within its block
  char* kt = nullptr;  // the block's K and V tiles (kv head g) in the pool
  char* vt = nullptr;

  // wave `wave` walks blocks j0 + wave + 4 i, i < nw, of the piece [j0, j1);
  // tbl holds the wave's first table entries (lane i: its block i)
  __device__ __forceinline__ void setup(const DecodeArgs& a, int b, int g, const SeqSpan& sp, int j0,
                                        int j1, int wave, int nw, int lane, int tbl) {
    const int last = sp.nb - 1;
    own = j1 == sp.nb && nw > 0 && j0 + wave + kWaves * (nw - 1) == last;
    if (!own) return;
    const int phys = nw <= kWave ? __builtin_amdgcn_readlane(tbl, nw - 1)
                                 : a.block_tables[(size_t)b * a.max_blocks_per_seq + sp.first_blk + last];
    // an unreadable block, or a length beyond max_context_len (its clamped
    // last position holds an older token): nothing to write
    if ((unsigned)phys >= (unsigned)a.num_blocks || sp.L_raw > a.max_context_len) {
      own = false;
      return;
    }
    const int Hkv = a.num_kv_heads;
    tn = (sp.L - 1) & (kBlock - 1);
    const size_t tile = ((size_t)phys * Hkv + g) * D * kBlock * ESZ;
    kt = reinterpret_cast<char*>(const_cast<void*>(a.k_pool)) + tile;
    vt = reinterpret_cast<char*>(const_cast<void*>(a.v_pool)) + tile;
    const size_t row = ((size_t)b * Hkv + g) * D * ESZ;
    const char* krow = reinterpret_cast<const char*>(a.k_new) + row;
    const char* vrow = reinterpret_cast<const char*>(a.v_new) + row;
    const int c = lane & 15, j = lane >> 4;
#pragma unroll
    for (int s = 0; s < KS; ++s) k[s] = *reinterpret_cast<const u32x4*>(krow + E * (4 * s + j) * ESZ);
    if constexpr (ESZ == 2) {
      const uint16_t* vr = reinterpret_cast<const uint16_t*>(vrow);
#pragma unroll
      for (int w = 0; w < VW; ++w)
        v[w] = (uint32_t)vr[32 * w + c] | ((uint32_t)vr[32 * w + 16 + c] << 16);
    } else {
      const uint32_t* vr = reinterpret_cast<const uint32_t*>(vrow);
#pragma unroll
      for (int x = 0; x < XT; ++x) v[x] = vr[16 * x + c];
    }
  }
  // raw bits of V dim 16 x + c
  __device__ __forceinline__ uint32_t vbits(int x) const {
    if constexpr (ESZ == 2)
      return (v[x >> 1] >> (16 * (x & 1))) & 0xFFFFu;
    else
      return v[x];
  }
  // K fragments: lanes of token tn take the new row
  template <typename V4>
  __device__ __forceinline__ void put_k(V4 (&kf)[KS], int lane) const {
    if ((lane & 15) == tn) {
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[s] = __builtin_bit_cast(V4, k[s]);
    }
  }
  // bf16 V fragments (tokens 4 j .. 4 j + 3 of dim 16 x + c, 16 bits each)
  __device__ __forceinline__ void put_v(u32x2 (&vf)[XT], int lane) const {
    if ((lane >> 4) == (tn >> 2)) {
      const int e = tn & 3, sh = 16 * (e & 1);
#pragma unroll
      for (int x = 0; x < XT; ++x) {
        const uint32_t keep = ~(0xFFFFu << sh), put = vbits(x) << sh;
        if (e < 2)
          vf[x].x = (vf[x].x & keep) | put;
        else
          vf[x].y = (vf[x].y & keep) | put;
      }
    }
  }
  // fp32 V fragments (tokens 4 j .. 4 j + 3 of dim 16 x + c)
  __device__ __forceinline__ void put_v(f32x4 (&vf)[XT], int lane) const {
    if ((lane >> 4) == (tn >> 2)) {
      const int e = tn & 3;
#pragma unroll
      for (int x = 0; x < XT; ++x) {
        const float nv = __builtin_bit_cast(float, vbits(x));
        vf[x].x = e == 0 ? nv : vf[x].x;
        vf[x].y = e == 1 ? nv : vf[x].y;
        vf[x].z = e == 2 ? nv : vf[x].z;
        vf[x].w = e == 3 ? nv : vf[x].w;
      }
    }
  }
  // the append itself: the rows into slot tn of the block
  __device__ __forceinline__ void store(int lane) const {
    const int c = lane & 15, j = lane >> 4;
    if (c == tn) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
        *reinterpret_cast<u32x4*>(kt + ((4 * s + j) * kBlock + tn) * 16) = k[s];
    }
    if (j == (tn >> 2)) {  // 16 lanes, one per c
#pragma unroll
      for (int x = 0; x < XT; ++x) {
        char* dst = vt + ((size_t)(16 * x + c) * kBlock + tn) * ESZ;
        if constexpr (ESZ == 2)
          *reinterpret_cast<uint16_t*>(dst) = (uint16_t)vbits(x);
        else
          *reinterpret_cast<uint32_t*>(dst) = vbits(x);
      }
    }
  }
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

// Merge the partials listed by `slots` for every query head of segment (b, g)
// and write the segment's output rows.  The G heads x D/4 float4 columns are
// spread over the threads; when they number fewer than the threads, the
// threads form `groups` copies of them and copy r takes the slots r,
// r + groups, ...  A thread issues the loads of up to kPer slots at once,
// then folds them into a running (max, sum, output); the copies are folded
// through LDS at the end.  All heads are merged in one pass, so the loads of
// the G rows are in flight together.
template <bool BF16, int D, typename SlotList, bool V = false>
__device__ void merge_segment(const DecodeArgs& a, int b, int g, SlotList slots, float* lds) {
  constexpr int kLanes = D / 4;  // float4 columns per row
  constexpr int kPer = 8;        // slots in flight per thread
  const int G = a.gqa_group;
  const int R = G * kLanes;      // (head, column) pairs
  const int groups = R >= kThreads ? 1 : kThreads / R;
  const int cnt = slots.count();
  const long long nsl = a.part_blocks > 0 ? (long long)a.num_seqs * a.num_kv_heads * a.num_partitions
                                          : 2LL * a.num_workers;
  const bool wide = nsl * G * D * 4 < (1LL << 31);
  const __amdgpu_buffer_rsrc_t ro = region(a.part_o, wide ? (int)(nsl * G * D * 4) : 0);
  for (int e0 = 0; e0 < R; e0 += kThreads) {
    const int e = groups > 1 ? (int)threadIdx.x % R : e0 + (int)threadIdx.x;
    const int grp = groups > 1 ? (int)threadIdx.x / R : 0;
    const bool active = e < R && grp < groups;
    const int h = e / kLanes, col = e % kLanes;
    float M = kNegInf, L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = grp; active && k0 < cnt; k0 += groups * kPer) {
      float mk[kPer], lk[kPer];
      f32x4 ov[kPer];
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        const int k = k0 + q * groups;
        int sl = 0;
        const bool valid = k < cnt && slots.slot(k, sl);
        lk[q] = 0.f;
        mk[q] = kNegInf;
        ov[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (valid) {
          mk[q] = load_dev(a.part_ml + ((size_t)sl * G + h) * 2);
          lk[q] = load_dev(a.part_ml + ((size_t)sl * G + h) * 2 + 1);
          const float* po = a.part_o + ((size_t)sl * G + h) * D + 4 * col;
          if (wide)
            ov[q] = load_dev4(ro, (int)((((size_t)sl * G + h) * D + 4 * col) * 4));
          else
            ov[q] = f32x4{load_dev(po), load_dev(po + 1), load_dev(po + 2), load_dev(po + 3)};
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
    if (groups > 1) {
      f32x4* lo = reinterpret_cast<f32x4*>(lds);  // [groups][R]
      float* lml = lds + 4 * groups * R;           // [groups][G][2]
      if (active) {
        lo[grp * R + e] = O;
        if (col == 0) {
          lml[2 * (grp * G + h)] = M;
          lml[2 * (grp * G + h) + 1] = L;
        }
      }
      __syncthreads();
      if (active && grp == 0) {
        float Mt = kNegInf;
        for (int q = 0; q < groups; ++q) Mt = fmaxf(Mt, lml[2 * (q * G + h)]);
        O = f32x4{0.f, 0.f, 0.f, 0.f};
        L = 0.f;
        if (Mt != kNegInf) {
          for (int q = 0; q < groups; ++q) {
            const float sc = fast_exp2(lml[2 * (q * G + h)] - Mt);
            O += lo[q * R + e] * sc;
            L += lml[2 * (q * G + h) + 1] * sc;
          }
        }
        M = Mt;
      }
    }
    if (active && grp == 0) finalize_vec<BF16, D>(a, b, g * G + h, 4 * col, O, L, M);
  }
}

// The four waves' (max, sum, output) of one piece, in LDS as lo[wave][head][D]
// and lml[wave][head][2]: merged, then written as the output (whole segment)
// or as the piece's partial.
template <bool BF16, int D, bool V = false>
__device__ void combine_waves(const DecodeArgs& a, const Piece& pc, const float* lo, const float* lml) {
  const int G = a.gqa_group;
  const int b = pc.b, g = pc.g;
  const SeqSpan& sp = pc.sp;
  const bool whole = (pc.j0 == 0 && pc.j1 == sp.nb);
  const int nvec = G * D / 4;
  // the piece's partial: O [G][D] and (max, sum) [G][2] at its slot
  const __amdgpu_buffer_rsrc_t ro = region(a.part_o + (size_t)pc.slot * G * D, G * D * 4);
  const __amdgpu_buffer_rsrc_t rml = region(a.part_ml + (size_t)pc.slot * G * 2, G * 8);
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
      store_dev4(ro, (h * D + d) * 4, O);
      if (d == 0) store_dev2(rml, h * 8, M, L);
    }
  }

}

// One block's logits of query row h for this lane's tokens tok .. tok + 3
// (base-2 logits s2, -inf where not visible), stored in natural-log units.
__device__ __forceinline__ void put_scores(const DecodeArgs& a, int b, int h, bool row_ok, int tok,
                                           const float (&s2)[4]) {
  if (!row_ok || a.scores == nullptr) return;  // sink tokens without logits: nothing to store
  const int Hq = a.num_kv_heads * a.gqa_group;
  float* dst = a.scores + ((size_t)b * Hq + h) * a.score_stride + tok;
  *reinterpret_cast<f32x4*>(dst) = f32x4{s2[0] * kLn2, s2[1] * kLn2, s2[2] * kLn2, s2[3] * kLn2};
}

// One piece: all four waves of the workgroup.
template <bool BF16, int D, bool FUSE, bool EVICT>
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

  // walk index j -> logical block (sink blocks first in the eviction variant)
  const SinkPart sk = EVICT ? sink_part(sp, a.window, a.sink) : SinkPart{0, 0};
  const int* bt = EVICT ? a.block_tables + (size_t)b * a.max_blocks_per_seq
                       : a.block_tables + (size_t)b * a.max_blocks_per_seq + sp.first_blk;
  const T* kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* vpool = reinterpret_cast<const T*>(a.v_pool);
  constexpr size_t kTile = (size_t)D * kBlock;

  // This wave's blocks: j0 + wave + 4 i, i < nw.  Their table entries are
  // read 64 at a time, one per lane, and picked out with readlane, so the
  // block loop itself touches memory only for K and V.
  const int span = pc.j1 - pc.j0 - wave;
  const int nw = span > 0 ? (span + kWaves - 1) / kWaves : 0;
  int tbl = 0;
  NewToken<sizeof(T), D> nt;
  if constexpr (FUSE) {
    const int t0 = nw > 0 ? a.block_tables[(size_t)b * a.max_blocks_per_seq + sp.first_blk + pc.j0 + wave +
                                           kWaves * min(lane, nw - 1)] : 0;
    nt.setup(a, b, g, sp, pc.j0, pc.j1, wave, nw, lane, t0);
  }

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
    const int tok0 = (EVICT ? sk.blk(sp, pc.j0 + wave + kWaves * i)
                            : sp.first_blk + pc.j0 + wave + kWaves * i) * kBlock;
    if constexpr (FUSE) {
      if (nt.own && i == nw - 1) {
        nt.put_k(buf.k, lane);
        nt.put_v(buf.v, lane);
        nt.store(lane);
      }
    }
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
      bool vis;
      if constexpr (EVICT)
        vis = ok & sk.visible(sp, t);
      else
        vis = ok & (t >= sp.vis_lo) & (t < sp.L);
      s2[r] = vis ? xf(sc[r]) : kNegInf;
    }
    if constexpr (EVICT) put_scores(a, b, g * G + c, c < G, tok0 + 4 * j, s2);
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
    if constexpr (EVICT)
      tbl = lane < cnt ? bt[sk.blk(sp, pc.j0 + wave + kWaves * (base + lane))] : 0;
    else
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

  combine_waves<BF16, D, EVICT>(a, pc, lo, lml);
  __syncthreads();  // LDS is reused by the next piece
}

// buffer resource of one block's K (or V) tile: a raw byte range, empty when
// the block may not be read (loads then return zeros)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_range(const void* base, int bytes) {
  constexpr unsigned kRawBufferWord3 = 0x00020000u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRawBufferWord3);
}

// The work of one cache block, bf16, with its K and V tiles in LDS at kt / vt
// (the pool's own layouts): S^T = K Q^T on the matrix cores, mask and logit
// transform, online softmax with lazy rescale, O^T += V^T P^T.  `newtok`: the
// block holds the fused append's new token (its rows are substituted and
// written to the pool).  The running state (o, m_run, l_run) is the caller's.
template <int D, bool FUSE, bool EVICT>
__device__ __forceinline__ void ring_block_step(const DecodeArgs& a, const LogitXform& xf,
                                                const char* kt, const char* vt, bool ok, int tok0,
                                                bool newtok, const NewToken<2, D>& nt,
                                                const SeqSpan& sp, const SinkPart& sk, int b, int g,
                                                const u32x4 (&qf)[D / 32], f32x4 (&o)[D / 16],
                                                float& m_run, float& l_run) {
  constexpr int KS = D / 32;  // score products
  constexpr int XT = D / 16;  // output tiles
  constexpr float kLazy = 8.0f;
  const int lane = threadIdx.x & 63, c = lane & 15, j = lane >> 4;
  const int G = a.gqa_group;
  u32x4 kf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) kf[s] = *reinterpret_cast<const u32x4*>(kt + (64 * s + lane) * 16);
  if constexpr (FUSE)
    if (newtok) nt.put_k(kf, lane);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) acc = mma_bf16_k32(kf[s], qf[s], acc);
  u32x2 vf[XT];
#pragma unroll
  for (int x = 0; x < XT; ++x)
    vf[x] = *reinterpret_cast<const u32x2*>(vt + (16 * x + c) * 2 * kBlock + 8 * j);
  if constexpr (FUSE) {
    if (newtok) {
      nt.put_v(vf, lane);
      nt.store(lane);
    }
  }
  mma_result_fence();

  float s2[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = tok0 + 4 * j + r;
    bool vis;
    if constexpr (EVICT)
      vis = ok & sk.visible(sp, t);
    else
      vis = ok & (t >= sp.vis_lo) & (t < sp.L);
    s2[r] = vis ? xf(acc[r]) : kNegInf;
  }
  if constexpr (EVICT) put_scores(a, b, g * G + c, c < G, tok0 + 4 * j, s2);
  float mx = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
  mx = quad_max(mx);
  if (__any(mx > m_run + kLazy)) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
    l_run *= alpha;
#pragma unroll
    for (int x = 0; x < XT; ++x) o[x] *= alpha;
    m_run = m_new;
  }
  const float m_use = m_run == kNegInf ? 0.f : m_run;
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s2[r] - m_use);
  l_run += (p[0] + p[1]) + (p[2] + p[3]);
  const u32x2 pa = {pack_bf16x2_hw(p[0], p[1]), pack_bf16x2_hw(p[2], p[3])};
  if (tok0 + kBlock > sp.L) {  // tokens past the context may hold anything
    const int nv = sp.L - tok0, t0 = 4 * j;
    const uint32_t mlo = (t0 + 0 < nv ? 0x0000FFFFu : 0u) | (t0 + 1 < nv ? 0xFFFF0000u : 0u);
    const uint32_t mhi = (t0 + 2 < nv ? 0x0000FFFFu : 0u) | (t0 + 3 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int x = 0; x < XT; ++x) vf[x] = u32x2{vf[x].x & mlo, vf[x].y & mhi};
  }
#pragma unroll
  for (int x = 0; x < XT; ++x) o[x] = mma_bf16_k16(vf[x], pa, o[x]);
}

// LDS bytes of the ring each wave of the LDS form streams its blocks through,
// and workgroups per CU: 32 KiB rings and one workgroup per CU at head_dim
// 128 and 256 (four and two blocks in flight per wave); at head_dim 64 two
// workgroups share a CU (16 KiB rings, four blocks in flight per wave), so
// one's start-up overlaps the other's streaming.
template <int D>
constexpr int kRingBytesPerWave = D >= 128 ? 32768 : 16384;
template <int D>
constexpr int kRingWgsPerCu = D >= 128 ? 1 : 2;

// The balanced split's price of one piece (its start, partial store and
// merge), in cache blocks of one kv head: PKV_DECODE_PIECE_COST_BYTES of K/V.
// split-K decode through the persistent kernel (0: one workgroup per partition)
#ifndef PKV_DECODE_FIXED_STREAM
#define PKV_DECODE_FIXED_STREAM 1
#endif
#ifndef PKV_DECODE_PIECE_COST_BYTES
#define PKV_DECODE_PIECE_COST_BYTES (192 * 1024)
#endif
template <int D>
constexpr int kPieceCost = PKV_DECODE_PIECE_COST_BYTES / (2 * kBlock * D * 2);

// One piece, bf16, blocks streamed through LDS.  Each wave walks its own
// blocks (j0 + wave + 4 i) with its own online softmax, O^T on the matrix
// cores, and the four waves are combined at the end.  K and V reach LDS by direct buffer-to-LDS copies into a ring private to
// the wave: NS = 32 KiB / (16 KiB x D / 256) blocks in flight per wave, with no
// vector registers held by loads and no barrier in the loop.  A block is
// copied verbatim (its K tile, then its V tile, 1 KiB per copy), so the
// operands are read with the pool's own layouts.
template <int D, bool FUSE, bool EVICT>
__device__ void run_piece_ring(const DecodeArgs& a, const LogitXform& xf, const Piece& pc,
                               float* lds) {
#ifdef PKV_TIMELINE
  if (pc.ord == 0) PKV_TL(a, 12);
  if (pc.ord == 1) PKV_TL(a, 14);
#endif
  constexpr int KS = D / 32;                        // score products
  constexpr int XT = D / 16;                        // output tiles
  constexpr int kTileBytes = D * kBlock * 2;        // one block's K (or V)
  constexpr int kRuns = 2 * kTileBytes / 1024;      // 1 KiB copies per block
  constexpr int NS = kRingBytesPerWave<D> / (2 * kTileBytes);
  static_assert(NS >= 2, "at least two blocks per wave in flight");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, j = lane >> 4;
  const int G = a.gqa_group, Hkv = a.num_kv_heads, Hq = G * Hkv;
  const int b = __builtin_amdgcn_readfirstlane(pc.b), g = __builtin_amdgcn_readfirstlane(pc.g);
  const int j0 = __builtin_amdgcn_readfirstlane(pc.j0), j1 = __builtin_amdgcn_readfirstlane(pc.j1);
  SeqSpan sp;
  sp.first_blk = __builtin_amdgcn_readfirstlane(pc.sp.first_blk);
  sp.nb = __builtin_amdgcn_readfirstlane(pc.sp.nb);
  sp.vis_lo = __builtin_amdgcn_readfirstlane(pc.sp.vis_lo);
  sp.L = __builtin_amdgcn_readfirstlane(pc.sp.L);
  sp.L_raw = __builtin_amdgcn_readfirstlane(pc.sp.L_raw);
  const SinkPart sk = EVICT ? sink_part(sp, a.window, a.sink) : SinkPart{0, 0};

  // query fragments: every lane loads from a real row (columns past the
  // group read its last row), then columns past the group are zeroed, so the
  // loads need no branches
  u32x4 qf[KS];
  {
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * Hq + g * G + min(c, G - 1)) * D + 8 * j;
    const uint32_t keep = c < G ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s) & keep;
  }

  f32x4 o[XT];
#pragma unroll
  for (int x = 0; x < XT; ++x) o[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const int span = j1 - j0 - wave;
  const int nw = span > 0 ? (span + kWaves - 1) / kWaves : 0;
  const int* bt = EVICT ? a.block_tables + (size_t)b * a.max_blocks_per_seq
                       : a.block_tables + (size_t)b * a.max_blocks_per_seq + sp.first_blk + j0 + wave;
  // table entry of this wave's block idx
  auto tbl_at = [&](int idx) { return EVICT ? bt[sk.blk(sp, j0 + wave + kWaves * idx)] : bt[kWaves * idx]; };
  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  char* ring = reinterpret_cast<char*>(lds) + wave * kRingBytesPerWave<D>;
  // this wave's table entries, 64 at a time (lane l: block tbase + l)
  int tbase = 0;
  int tbl = lane < nw ? tbl_at(lane) : 0;
  NewToken<2, D> nt;
  if constexpr (FUSE) nt.setup(a, b, g, sp, j0, j1, wave, nw, lane, tbl);
  uint32_t okbits = 0;  // bit (block % NS): that slot's block was readable
#ifdef PKV_TIMELINE
  if (pc.ord == 0) {
    PKV_TL(a, 13);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    PKV_TL(a, 16);
  }
#endif

  // copy this wave's block i (past the end: an empty range, zeros) into its slot
  auto issue = [&](int i) {
    if (i - tbase >= 64) {  // uniform, every 64 blocks
      tbase += 64;
      tbl = tbase + lane < nw ? tbl_at(tbase + lane) : 0;
    }
    const int phys = __builtin_amdgcn_readlane(tbl, (i - tbase) & 63);
    const bool ok = i < nw && (unsigned)phys < (unsigned)a.num_blocks;
    const size_t off = ((size_t)(ok ? phys : 0) * Hkv + g) * kTileBytes;
    const __amdgpu_buffer_rsrc_t rk = tile_range(kpool + off, ok ? kTileBytes : 0);
    const __amdgpu_buffer_rsrc_t rv = tile_range(vpool + off, ok ? kTileBytes : 0);
    const int slot = i % NS;
    okbits = (okbits & ~(1u << slot)) | ((uint32_t)ok << slot);
    char* dst = ring + slot * 2 * kTileBytes;
#pragma unroll
    for (int r = 0; r < kRuns / 2; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(dst + r * 1024),
                                               16, r * 1024 + lane * 16, 0, 0, kStreamLoad);
#pragma unroll
    for (int r = 0; r < kRuns / 2; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(dst + kTileBytes + r * 1024),
                                               16, r * 1024 + lane * 16, 0, 0, kStreamLoad);
  };

#pragma unroll
  for (int i = 0; i < NS; ++i) issue(i);
#ifdef PKV_TIMELINE
  if (pc.ord == 0) PKV_TL(a, 2);
  if (pc.ord == 1) PKV_TL(a, 15);
#endif
  for (int i = 0; i < nw; ++i) {
    // block i has landed: the NS - 1 later blocks may still be in flight
    constexpr int kAfter = (NS - 1) * kRuns;
    __builtin_amdgcn_s_waitcnt((kAfter & 15) | ((kAfter >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
#ifdef PKV_TIMELINE
    if (pc.ord == 0 && i == 0) PKV_TL(a, 3);
#endif
    const int slot = i % NS;
    const bool ok = (okbits >> slot) & 1u;
    const char* kt = ring + slot * 2 * kTileBytes;
    const char* vt = kt + kTileBytes;
    const int tok0 =
        (EVICT ? sk.blk(sp, j0 + wave + kWaves * i) : sp.first_blk + j0 + wave + kWaves * i) * kBlock;

    const bool newtok = FUSE && nt.own && i == nw - 1;
    ring_block_step<D, FUSE, EVICT>(a, xf, kt, vt, ok, tok0, newtok, nt, sp, sk, b, g, qf, o, m_run,
                                    l_run);
    asm volatile("" ::: "memory");
    issue(i + NS);  // into the slot just read (the products have their operands)
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the copies past the end have landed
  PKV_TL_WAVE(a, 4);

  // ---- combine the four waves through LDS (the rings are free now) ----
  mma_result_fence();
  const float l_tot = quad_sum(l_run);
  __syncthreads();
  PKV_TL(a, 17);
  float* lo = lds;                    // [4][G][D]
  float* lml = lds + kWaves * G * D;  // [4][G][2]
  if (c < G) {
#pragma unroll
    for (int x = 0; x < XT; ++x)
      *reinterpret_cast<f32x4*>(lo + ((size_t)wave * G + c) * D + 16 * x + 4 * j) = o[x];
    if (j == 0) {
      lml[(wave * G + c) * 2] = m_run;
      lml[(wave * G + c) * 2 + 1] = l_tot;
    }
  }
  __syncthreads();
  PKV_TL(a, 18);
  combine_waves<true, D, EVICT>(a, pc, lo, lml);
  __syncthreads();  // LDS is reused by the next piece
  PKV_TL(a, 8);
}

// ---------------------------------------------------------------------------
// Split-K decode (fixed partitions), persistent form.  One workgroup per CU
// takes a contiguous run of the (segment, partition) items -- the visible
// partitions of every segment, segment after segment -- and streams their
// blocks through per-wave LDS rings that carry over from one partition to the
// next: while a partition is combined and its partial stored, the next one's
// first blocks are already being copied.  A workgroup counts its partitions
// of a segment in with one atomic add when it leaves the segment; the one
// that completes the count merges the segment.  The result is the same as
// one workgroup per partition (same partials, same merge), without a round of
// workgroup start-ups per partition.
// ---------------------------------------------------------------------------
// per wave: two blocks in flight at head_dim 256 and 128 (four at 64).  At
// head_dim 128 a 32 KiB ring (four blocks) measured 1.3% slower on the long-
// context split-K shape: with every CU streaming, fewer bytes in flight per CU
// serve the memory system better.
template <int D>
constexpr int kStreamRingBytes = D >= 256 ? 32768 : 16384;
constexpr int kDummyBytes = 1024;        // takes the empty prologue copies
template <int D>
__host__ __device__ constexpr int combine_bytes(int G) {
  return kWaves * G * (D + 2) * 4 > (4 * kThreads + 2 * 16) * 4 ? kWaves * G * (D + 2) * 4
                                                                  : (4 * kThreads + 2 * 16) * 4;
}
template <int D>
__host__ __device__ constexpr int fixed_stream_lds(int G) {
  return kWaves * kStreamRingBytes<D> + combine_bytes<D>(G) + kDummyBytes;
}
constexpr int kLdsPerCu = 163840;

// A wave's LDS ring carried from one partition to the next.  Block k of the
// current partition sits at stream position pos + k, ring slot (pos + k) % NS.
// When the next partition gives this wave at least NS blocks, the current one
// loads its table slice and query fragments when it starts and issues its
// first NS blocks in its own last NS steps.
template <int D>
struct RingStream {
  int pos = 0;
  uint32_t okbits = 0;  // bit (position % NS): that slot's block was readable
  bool pre = false;     // the current partition's first NS blocks are issued
  bool qpre = false;    // its query fragments are in qn
  int tbl = 0;          // its table slice (lane l: block l of this wave), if pre
  u32x4 qn[D / 32];
};

// One partition (a piece of a segment), bf16, through the carried rings; the
// per-block work is that of run_piece_ring.  The waves are combined in the
// region beside the rings (cmb), followed by the dummy KiB.
template <int D, bool FUSE>
__device__ void run_piece_stream(const DecodeArgs& a, const LogitXform& xf, const Piece& pc,
                                 const Piece& nx, bool has_nx, RingStream<D>& rs, float* lds,
                                 float* cmb) {
  constexpr int KS = D / 32;                        // score products
  constexpr int XT = D / 16;                        // output tiles
  constexpr int kTileBytes = D * kBlock * 2;        // one block's K (or V)
  constexpr int kRuns = 2 * kTileBytes / 1024;      // 1 KiB copies per block
  constexpr int NS = kStreamRingBytes<D> / (2 * kTileBytes);
  static_assert(NS >= 2 && (NS & (NS - 1)) == 0, "a power of two, at least two blocks in flight");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, j = lane >> 4;
  const int G = a.gqa_group, Hkv = a.num_kv_heads, Hq = G * Hkv;
  const int b = __builtin_amdgcn_readfirstlane(pc.b), g = __builtin_amdgcn_readfirstlane(pc.g);
  const int j0 = __builtin_amdgcn_readfirstlane(pc.j0), j1 = __builtin_amdgcn_readfirstlane(pc.j1);
  SeqSpan sp;
  sp.first_blk = __builtin_amdgcn_readfirstlane(pc.sp.first_blk);
  sp.nb = __builtin_amdgcn_readfirstlane(pc.sp.nb);
  sp.vis_lo = __builtin_amdgcn_readfirstlane(pc.sp.vis_lo);
  sp.L = __builtin_amdgcn_readfirstlane(pc.sp.L);
  sp.L_raw = __builtin_amdgcn_readfirstlane(pc.sp.L_raw);
  const int span = j1 - j0 - wave;
  const int nw = span > 0 ? (span + kWaves - 1) / kWaves : 0;

  // the carried state is the same in every lane: keep it scalar, so the ring
  // addresses and the load descriptors stay scalar
  has_nx = __builtin_amdgcn_readfirstlane((int)has_nx) != 0;
  const bool pre = __builtin_amdgcn_readfirstlane((int)rs.pre) != 0;
  const bool qpre = __builtin_amdgcn_readfirstlane((int)rs.qpre) != 0;
  int nb_ = 0, ng = 0, nj0 = 0, nnw = 0, nfirst = 0;
  if (has_nx) {
    nb_ = __builtin_amdgcn_readfirstlane(nx.b);
    ng = __builtin_amdgcn_readfirstlane(nx.g);
    nj0 = __builtin_amdgcn_readfirstlane(nx.j0);
    const int nj1 = __builtin_amdgcn_readfirstlane(nx.j1);
    nfirst = __builtin_amdgcn_readfirstlane(nx.sp.first_blk);
    const int nspan = nj1 - nj0 - wave;
    nnw = nspan > 0 ? (nspan + kWaves - 1) / kWaves : 0;
  }
  const bool pf = has_nx && nnw >= NS;  // prefetch the next partition's first blocks

  const int* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq + sp.first_blk + j0 + wave;
  const int* nbt = a.block_tables + (size_t)nb_ * a.max_blocks_per_seq + nfirst + nj0 + wave;
  int tbase = 0;
  int tbl = pre ? rs.tbl : (lane < nw ? bt[kWaves * lane] : 0);
  const int ntbl = pf && lane < nnw ? nbt[kWaves * lane] : 0;

  u32x4 qf[KS];
  if (qpre) {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = rs.qn[s];
  } else {
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * Hq + g * G + min(c, G - 1)) * D + 8 * j;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s) & (c < G ? 0xFFFFFFFFu : 0u);
  }
  if (has_nx) {
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(a.q) + ((size_t)nb_ * Hq + ng * G + min(c, G - 1)) * D + 8 * j;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      rs.qn[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s) & (c < G ? 0xFFFFFFFFu : 0u);
  }
  NewToken<2, D> nt;
  if constexpr (FUSE) nt.setup(a, b, g, sp, j0, j1, wave, nw, lane, tbl);

  f32x4 o[XT];
#pragma unroll
  for (int x = 0; x < XT; ++x) o[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  char* ring = reinterpret_cast<char*>(lds) + wave * kStreamRingBytes<D>;
  char* dummy = reinterpret_cast<char*>(cmb) + combine_bytes<D>(G);
  const int pos = __builtin_amdgcn_readfirstlane(rs.pos);
  uint32_t okbits = __builtin_amdgcn_readfirstlane(rs.okbits);

  // stream entry k of this partition: its block k, then (when prefetching)
  // the next partition's blocks 0 .. NS - 1, then empty ranges (zeros).
  // `fake`: an empty copy into the dummy KiB that takes no stream position.
  auto issue = [&](int k, bool fake) {
    int phys = 0, gg = g;
    bool ok = false;
    if (fake) {
    } else if (k < nw) {
      if (k - tbase >= 64) {  // uniform, every 64 blocks
        tbase += 64;
        tbl = tbase + lane < nw ? bt[kWaves * (tbase + lane)] : 0;
      }
      phys = __builtin_amdgcn_readlane(tbl, (k - tbase) & 63);
      ok = (unsigned)phys < (unsigned)a.num_blocks;
    } else if (pf && k - nw < NS) {
      phys = __builtin_amdgcn_readlane(ntbl, (k - nw) & 63);
      gg = ng;
      ok = (unsigned)phys < (unsigned)a.num_blocks;
    }
    const size_t off = ((size_t)(ok ? phys : 0) * Hkv + gg) * kTileBytes;
    const __amdgpu_buffer_rsrc_t rk = tile_range(kpool + off, ok ? kTileBytes : 0);
    const __amdgpu_buffer_rsrc_t rv = tile_range(vpool + off, ok ? kTileBytes : 0);
    const int slot = (pos + k) & (NS - 1);
    if (!fake) okbits = (okbits & ~(1u << slot)) | ((uint32_t)ok << slot);
    char* dst = fake ? dummy : ring + slot * 2 * kTileBytes;
    const int step = fake ? 0 : 1024;  // a fake copy's runs all land on the dummy KiB
#pragma unroll
    for (int r = 0; r < kRuns / 2; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(dst + r * step),
                                               16, r * 1024 + lane * 16, 0, 0, kStreamLoad);
#pragma unroll
    for (int r = 0; r < kRuns / 2; ++r)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void*)(dst + (fake ? 0 : kTileBytes) + r * step), 16,
          r * 1024 + lane * 16, 0, 0, kStreamLoad);
  };

  // NS prologue copies on every path (fake ones when the partition before
  // issued this one's first blocks): the loop is then entered the same way
  // whatever came before it, and its waits hold NS - 1 copies or more after
  // each block.
#pragma unroll
  for (int k = 0; k < NS; ++k) issue(k, pre);
  for (int i = 0; i < nw; ++i) {
    // block i has landed: at least NS - 1 later stream entries were issued after it
    constexpr int kAfter = (NS - 1) * kRuns;
    __builtin_amdgcn_s_waitcnt((kAfter & 15) | ((kAfter >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
    const int slot = (pos + i) & (NS - 1);
    const bool ok = (okbits >> slot) & 1u;
    const char* kt = ring + slot * 2 * kTileBytes;
    const char* vt = kt + kTileBytes;
    const int tok0 = (sp.first_blk + j0 + wave + kWaves * i) * kBlock;

    const bool newtok = FUSE && nt.own && i == nw - 1;
    ring_block_step<D, FUSE, false>(a, xf, kt, vt, ok, tok0, newtok, nt, sp, SinkPart{0, 0}, b, g, qf,
                                    o, m_run, l_run);
    asm volatile("" ::: "memory");
    issue(i + NS, false);  // into the slot just read (the products have their operands)
  }
  // without a prefetch, let the copies past the end land (the next
  // partition's prologue reuses the slots)
  if (!pf) __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- combine the four waves beside the rings ----
  mma_result_fence();
  const float l_tot = quad_sum(l_run);
  float* lo = cmb;                    // [4][G][D]
  float* lml = lo + kWaves * G * D;   // [4][G][2]
  if (c < G) {
#pragma unroll
    for (int x = 0; x < XT; ++x)
      *reinterpret_cast<f32x4*>(lo + ((size_t)wave * G + c) * D + 16 * x + 4 * j) = o[x];
    if (j == 0) {
      lml[(wave * G + c) * 2] = m_run;
      lml[(wave * G + c) * 2 + 1] = l_tot;
    }
  }
  __syncthreads();
  combine_waves<true, D, false>(a, pc, lo, lml);
  __syncthreads();  // the combine region is reused next

  rs.pos = pos + nw;
  rs.okbits = okbits;
  rs.pre = pf;
  rs.tbl = ntbl;
  rs.qpre = has_nx;
}

// Output of a sequence with nothing to attend to: 0, lse = -inf.
template <bool BF16, int D, bool V = false>
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

// k pieces of a split segment have stored their partials: count them in; the
// workgroup that counts the last piece merges all of them into the output
// and resets the counter (the counters start at zero and are left at zero).
template <bool BF16, int D, bool V, typename SlotList>
__device__ void finish_split(const DecodeArgs& a, int b, int g, SlotList slots, float* lds, int k = 1) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial stores are done
  __syncthreads();
  PKV_TL(a, 19);
  int* cnt = a.seg_count + (size_t)b * a.num_kv_heads + g;
  int* flag = reinterpret_cast<int*>(lds);
  if (threadIdx.x == 0)
    flag[0] = __hip_atomic_fetch_add(cnt, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == slots.count() - k;
  __syncthreads();
  const bool last = flag[0] != 0;
  __syncthreads();  // LDS is reused below
  PKV_TL(a, 9);
  if (!last) return;
  merge_segment<BF16, D, SlotList, V>(a, b, g, slots, lds);
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  PKV_TL(a, 10);
}

// Split-K decode, persistent form (see run_piece_stream): workgroup w of N
// takes items [w I / N, (w + 1) I / N) of the I (segment, partition) items.
template <int D, bool FUSE>
__global__ __launch_bounds__(kThreads, 1) void decode_fixed_stream_kernel(DecodeArgs a) {
  extern __shared__ float lds[];
  const LogitXform xf = make_xform(a.scale, a.softcap);
  const int Hkv = a.num_kv_heads, G = a.gqa_group, B = a.num_seqs;
  const int NP = a.num_partitions, PB = a.part_blocks;
  const int N = gridDim.x, w = blockIdx.x;
  const int lane = threadIdx.x & 63;
  float* cmb = lds + kWaves * kStreamRingBytes<D> / 4;
  auto span = [&](int L) { return seq_span(L, a.window, a.max_context_len); };
  // visible partitions of a sequence of length L
  auto parts = [&](int L) -> int {
    const SeqSpan sp = span(L);
    return sp.nb > 0 ? (sp.first_blk + sp.nb - 1) / PB - sp.first_blk / PB + 1 : 0;
  };

  // context lengths of sequences 64 r + lane, r < kLenRegs, in registers
  constexpr int kLenRegs = 4;
  int Lr[kLenRegs];
#pragma unroll
  for (int r = 0; r < kLenRegs; ++r) {
    const int b = r * kWave + lane;
    Lr[r] = b < B ? a.context_lens[b] : 0;
  }
  auto len_at = [&](int r) -> int {  // length of sequence 64 r + lane (0 past B)
    int L = 0;
#pragma unroll
    for (int q = 0; q < kLenRegs; ++q) L = q == r ? Lr[q] : L;
    if (r >= kLenRegs) {
      const int b = r * kWave + lane;
      L = b < B ? a.context_lens[b] : 0;
    }
    return L;
  };
  auto len_of = [&](int b) -> int {  // length of sequence b (uniform)
    return b < kLenRegs * kWave ? __builtin_amdgcn_readlane(len_at(b / kWave), b % kWave)
                                : a.context_lens[b];
  };

  for (int b = w; b < B; b += N)  // sequences with no visible token
    if (span(len_of(b)).nb == 0) write_empty<true, D, false>(a, b, 0, Hkv * G);

  long long I = 0, i0 = 0, i1 = 0, seg_base = 0;
  int b0 = 0;
  if (B <= kLenRegs * kWave && a.units32) {
    // as the balanced split's set-up: one DPP scan per 64 sequences
    int incl[kLenRegs], tot[kLenRegs], own[kLenRegs];
#pragma unroll
    for (int r = 0; r < kLenRegs; ++r) {
      incl[r] = tot[r] = own[r] = 0;
      if (r * kWave < B) {
        own[r] = parts(Lr[r]) * Hkv;
        incl[r] = wave_incl_scan_i32(own[r]);
        tot[r] = __builtin_amdgcn_readlane(incl[r], kWave - 1);
        I += tot[r];
      }
    }
    i0 = __builtin_amdgcn_readfirstlane((long long)w * I / N);
    i1 = (long long)(w + 1) * I / N;
    if (i0 >= i1) return;
    long long run = 0;
#pragma unroll
    for (int r = 0; r < kLenRegs; ++r) {
      if (r * kWave >= B) break;
      const unsigned long long hit = __ballot(run + incl[r] > i0);
      if (hit) {
        const int l0 = __ffsll(hit) - 1;
        b0 = r * kWave + l0;
        seg_base = run + __builtin_amdgcn_readlane(incl[r] - own[r], l0);
        break;
      }
      run += tot[r];
    }
  } else {
    for (int r = 0; r * kWave < B; ++r) I += wave_sum_i64(parts(len_at(r)));
    I *= Hkv;
    i0 = __builtin_amdgcn_readfirstlane((long long)w * I / N);
    i1 = (long long)(w + 1) * I / N;
    if (i0 >= i1) return;
    // segment holding item i0: first sequence whose inclusive prefix exceeds i0
    long long run = 0;
    for (int r = 0; r * kWave < B; ++r) {
      const long long nph = (long long)parts(len_at(r)) * Hkv;
      const long long incl = wave_incl_scan_i64(nph, lane);
      const unsigned long long hit = __ballot(run + incl > i0);
      if (hit) {
        const int l0 = __ffsll(hit) - 1;
        b0 = r * kWave + l0;
        seg_base = run + __shfl(incl - nph, l0);
        break;
      }
      run += __shfl(incl, kWave - 1);
    }
  }
  seg_base = __builtin_amdgcn_readfirstlane(seg_base);

  // The pieces of [i0, i1): runs of consecutive partitions of one segment.
  // A run is walked as one piece (its partitions' partials are folded as the
  // blocks stream: the online softmax over a run of partitions is the
  // log-sum-exp merge of their partials) and stored at the slot of its first
  // partition.  Cursor: sequence cb, kv head cg, partition index cp (from the
  // first visible one) and the segment's first item S.
  int cb = b0;
  SeqSpan csp = span(len_of(cb));
  int cnp = parts(csp.L);
  const int r0 = (int)(i0 - seg_base);
  int cg = r0 / cnp, cp = r0 % cnp;
  long long S = seg_base + (long long)cg * cnp;
  long long left = i1 - i0;
  auto next_piece = [&](Piece& out) -> bool {
    if (left <= 0) return false;
    const int run_len = (int)min((long long)(cnp - cp), left);
    const int p_lo = csp.first_blk / PB, p = p_lo + cp;
    const int lo = max(p * PB, csp.first_blk);
    const int hi = min((p + run_len) * PB, csp.first_blk + csp.nb);
    out.b = cb;
    out.g = cg;
    out.sp = csp;
    out.j0 = lo - csp.first_blk;
    out.j1 = hi - csp.first_blk;
    out.slot = (cb * Hkv + cg) * NP + p;
    out.S = S;
    left -= run_len;
    cp += run_len;
    if (left > 0) {  // the run ended with its segment: move to the next one
      S += cnp;
      cp = 0;
      if (++cg == Hkv) {
        cg = 0;
        do {
          ++cb;
          csp = span(len_of(cb));
          cnp = parts(csp.L);
        } while (cnp == 0);
      }
    }
    return true;
  };

  RingStream<D> rs;
  Piece cur;
  bool has = __builtin_amdgcn_readfirstlane((int)next_piece(cur)) != 0;
  while (has) {
    Piece nxt = cur;
    const bool has_n = __builtin_amdgcn_readfirstlane((int)next_piece(nxt)) != 0;
    run_piece_stream<D, FUSE>(a, xf, cur, nxt, has_n, rs, lds, cmb);
    if (!(cur.j0 == 0 && cur.j1 == cur.sp.nb)) {
      const int seg = cur.b * Hkv + cur.g;
      const int p_lo = cur.sp.first_blk / PB;
      const long long nparts = parts(cur.sp.L);
      finish_split<true, D, false>(a, cur.b, cur.g,
                                   RunSlots{I, cur.S, cur.S + nparts, N, seg * NP + p_lo}, cmb);
    }
    cur = nxt;
    has = has_n;
  }
}

// The decode of workgroup `blk` (of num_workers in the balanced split, of
// the (segment, partition) grid in the fixed one), with `lds` the
// workgroup's dynamic LDS.  decode_kernel runs it for its own workgroup; the
// mixed-batch kernel runs it for the workgroups after the prefill's.
template <bool BF16, int D, bool FIXED, bool FUSE, bool EVICT>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, int blk, float* lds) {
  auto run_one = [&](const LogitXform& xf, const Piece& pc) {
    if constexpr (BF16) {
      run_piece_ring<D, FUSE, EVICT>(a, xf, pc, lds);
    } else {
      run_piece<BF16, D, FUSE, EVICT>(a, xf, pc, lds);
    }
  };
  const LogitXform xf = make_xform(a.scale, a.softcap);
  const int Hkv = a.num_kv_heads, G = a.gqa_group;
  // a sequence's visible span (with the sink tokens in the eviction variant)
  auto span = [&](int L_raw) {
    if constexpr (EVICT)
      return seq_span_sink(L_raw, a.window, a.max_context_len, a.sink);
    else
      return seq_span(L_raw, a.window, a.max_context_len);
  };

  if constexpr (FIXED) {
    const int NP = a.num_partitions, PB = a.part_blocks;
    const int seg = blk / NP, p = blk % NP;
    const int b = seg / Hkv, g = seg % Hkv;
    Piece pc;
    pc.b = b;
    pc.g = g;
    pc.sp = seq_span(a.context_lens[b], a.window, a.max_context_len);
    if (pc.sp.nb == 0) {
      if (p == 0) write_empty<BF16, D, EVICT>(a, b, g * G, (g + 1) * G);
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
    if (!(pc.j0 == 0 && pc.j1 == pc.sp.nb)) {
      const int p_lo = pc.sp.first_blk / PB, p_hi = last_blk / PB;
      finish_split<BF16, D, EVICT>(a, b, g, SplitSlots{seg * NP, p_lo, p_hi}, lds);
    }
  } else {
    const int N = a.num_workers, w = blk;
    const int lane = threadIdx.x & 63;
    const int B = a.num_seqs;
    PKV_TL(a, 0);
#ifdef PKV_TIMELINE
    int tl_pieces = 0;
#endif

    // Context lengths of sequences 64 r + lane, r < kLenRegs, held in
    // registers: one load for the whole set-up below (the work total, the
    // scan for this workgroup's first segment, its span and the empty
    // sequences), so that the chain before the first K/V copies is the
    // lengths, then the block table.  Longer batches read the rest as needed.
    constexpr int kLenRegs = 4;
    int Lr[kLenRegs];
#pragma unroll
    for (int r = 0; r < kLenRegs; ++r) {
      const int b = r * kWave + lane;
      Lr[r] = b < B ? a.context_lens[b] : 0;
    }
    auto len_at = [&](int r) -> int {  // length of sequence 64 r + lane (0 past B)
      int L = 0;
#pragma unroll
      for (int q = 0; q < kLenRegs; ++q) L = q == r ? Lr[q] : L;
      if (r >= kLenRegs) {
        const int b = r * kWave + lane;
        L = b < B ? a.context_lens[b] : 0;
      }
      return L;
    };

    // sequences with no visible token
    for (int b = w; b < B; b += N) {
      const int L = __builtin_amdgcn_readlane(len_at(b / kWave), b % kWave);
      if (span(L).nb == 0) write_empty<BF16, D, EVICT>(a, b, 0, Hkv * G);
    }

    // The split runs over W = sum of (kPieceCost<D> + nb) x Hkv units: every
    // segment's nb real units preceded by kPieceCost<D> units that stand for
    // the fixed cost of a piece (its start, partial store and merge), so that
    // a workgroup whose range crosses into another segment takes fewer real
    // units.  Every wave computes the same W.
    constexpr int C = kPieceCost<D>;
    auto seg_units = [&](int nb) -> long long { return nb > 0 ? (long long)(nb + C) : 0; };
    long long W = 0, a0 = 0, a1 = 0, seg_base = 0;
    int b0 = 0, L0 = 0;
    if (B <= kLenRegs * kWave && a.units32) {
      // the lengths are all in registers and every total fits in 31 bits:
      // one DPP scan per 64 sequences gives both the work total and, with a
      // ballot, the segment holding unit a0 (no LDS round trips)
      int incl[kLenRegs], tot[kLenRegs];
#pragma unroll
      for (int r = 0; r < kLenRegs; ++r) {
        incl[r] = tot[r] = 0;
        if (r * kWave < B) {
          incl[r] = wave_incl_scan_i32((int)seg_units(span(Lr[r]).nb) * Hkv);
          tot[r] = __builtin_amdgcn_readlane(incl[r], kWave - 1);
          W += tot[r];
        }
      }
      a0 = (long long)w * W / N;
      a1 = (long long)(w + 1) * W / N;
      if (a0 >= a1) return;
      long long run = 0;
#pragma unroll
      for (int r = 0; r < kLenRegs; ++r) {
        if (r * kWave >= B) break;
        const unsigned long long hit = __ballot(run + incl[r] > a0);
        if (hit) {
          const int l0 = __ffsll(hit) - 1;
          b0 = r * kWave + l0;
          L0 = __builtin_amdgcn_readlane(Lr[r], l0);
          const int own = (int)seg_units(span(L0).nb) * Hkv;
          seg_base = run + __builtin_amdgcn_readlane(incl[r], l0) - own;
          break;
        }
        run += tot[r];
      }
    } else {
      for (int r = 0; r * kWave < B; ++r) W += wave_sum_i64(seg_units(span(len_at(r)).nb));
      W *= Hkv;
      a0 = (long long)w * W / N;
      a1 = (long long)(w + 1) * W / N;
      if (a0 >= a1) return;
      // segment holding unit a0: first sequence whose inclusive prefix exceeds a0
      long long run = 0;
      for (int r = 0; r * kWave < B; ++r) {
        const int Lb = len_at(r);
        const long long nbh = seg_units(span(Lb).nb) * Hkv;
        const long long incl = wave_incl_scan_i64(nbh, lane);
        const unsigned long long hit = __ballot(run + incl > a0);
        if (hit) {
          const int l0 = __ffsll(hit) - 1;
          b0 = r * kWave + l0;
          L0 = __builtin_amdgcn_readlane(Lb, l0);
          seg_base = run + __shfl(incl - nbh, l0);
          break;
        }
        run += __shfl(incl, kWave - 1);
      }
    }

    Piece pc;
    pc.b = b0;
    pc.sp = span(L0);
    pc.g = (int)((a0 - seg_base) / (pc.sp.nb + C));
    long long Sv = seg_base + (long long)pc.g * (pc.sp.nb + C);  // segment start (cost units)
    bool first = true;
    PKV_TL(a, 1);
    while (true) {
      const long long S = Sv + C, E = S + pc.sp.nb;  // the segment's real units
      const long long lo = max(a0, S), hi = min(a1, E);
      if (lo < hi) {
        pc.S = S;
        pc.j0 = (int)(lo - S);
        pc.j1 = (int)(hi - S);
        pc.slot = first ? 2 * w : 2 * w + 1;
#ifdef PKV_TIMELINE
        pc.ord = tl_pieces++;
#endif
        run_one(xf, pc);
        if (!(pc.j0 == 0 && pc.j1 == pc.sp.nb))
          finish_split<BF16, D, EVICT>(a, pc.b, pc.g, BalancedSlots{W, S, E, Sv, N}, lds);
      }
      first = false;
      Sv = E;
      if (Sv >= a1) break;
      if (++pc.g == Hkv) {
        pc.g = 0;
        do {
          if (++pc.b >= B) break;
          pc.sp = span(a.context_lens[pc.b]);
        } while (pc.sp.nb == 0);
        if (pc.b >= B) break;
      }
    }
    PKV_TL(a, 11);
  }
}

template <bool BF16, int D, bool FIXED, bool FUSE, bool EVICT>
__global__ __launch_bounds__(kThreads, !BF16 ? 1 : kRingWgsPerCu<D>) void decode_kernel(DecodeArgs a) {
  extern __shared__ float lds[];
  decode_body<BF16, D, FIXED, FUSE, EVICT>(a, blockIdx.x, lds);
}

// H2O statistic of the decode step: mass[b, g, t] = sum over the group's
// query heads h of exp(logit[b, h, t] - lse[b, h]), the softmax weight of
// token t, for visible t; 0 elsewhere in the row.  One thread per token.
__global__ __launch_bounds__(kThreads) void column_mass_kernel(DecodeArgs a) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= a.score_stride) return;
  const int seg = blockIdx.y, Hkv = a.num_kv_heads, G = a.gqa_group;
  const int b = seg / Hkv, g = seg % Hkv;
  const SeqSpan sp = seq_span(a.context_lens[b], a.window, a.max_context_len);
  const SinkPart sk = sink_part(sp, a.window, a.sink);
  float mass = 0.f;
  if (sk.visible(sp, t)) {
    const size_t row0 = (size_t)b * Hkv * G + (size_t)g * G;
    for (int h = 0; h < G; ++h)
      mass += fast_exp2((a.scores[(row0 + h) * a.score_stride + t] - a.lse[row0 + h]) * kLog2e);
  }
  a.column_mass[(size_t)seg * a.score_stride + t] = mass;
}

// The combine buffer holds the four waves' partial outputs: up to 66 KiB for
// a group of 16 at head_dim 256, above the default 64 KiB dynamic-LDS limit.
template <typename K>
hipError_t allow_lds(K kernel, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <typename K>
hipError_t launch_k(K kernel, const DecodeArgs& a, size_t lds, hipStream_t stream) {
  hipError_t e = allow_lds(kernel, lds);
  if (e != hipSuccess) return e;
  kernel<<<a.num_workers, kThreads, lds, stream>>>(a);
  return hipGetLastError();
}

// Balanced-split grid: workgroups per CU, and a floor on the blocks a
// workgroup gets (tiny batches use fewer workgroups).
#ifndef PKV_DECODE_WGS_PER_CU
#define PKV_DECODE_WGS_PER_CU 1
#endif
#ifndef PKV_DECODE_MIN_BLOCKS_PER_WG
#define PKV_DECODE_MIN_BLOCKS_PER_WG 8
#endif

template <bool BF16, int D>
hipError_t launch_d(DecodeArgs a, hipStream_t stream) {
  if (a.part_blocks == 0) {
    long long n = (a.units_bound + PKV_DECODE_MIN_BLOCKS_PER_WG - 1) / PKV_DECODE_MIN_BLOCKS_PER_WG;
    const long long cap =
        (long long)a.cu_count * (!BF16 ? PKV_DECODE_WGS_PER_CU : kRingWgsPerCu<D>);
    n = min(n, min(cap, (long long)kMaxWorkers));
    a.num_workers = (int32_t)max(n, 1LL);
  }
  size_t lds = (size_t)kWaves * a.gqa_group * (D + 2) * sizeof(float);  // the waves' combine
  lds = std::max(lds, (size_t)(4 * kThreads + 2 * 16) * sizeof(float));  // a merge
  if (BF16) lds = std::max(lds, (size_t)kWaves * kRingBytesPerWave<D>);
  if (a.part_blocks > 0) {
    if constexpr (BF16) {
      if (PKV_DECODE_FIXED_STREAM && fixed_stream_lds<D>(a.gqa_group) <= kLdsPerCu) {
        // persistent form: one workgroup per CU, at most one per item
        DecodeArgs p = a;
        const long long items = (long long)a.num_seqs * a.num_kv_heads * a.num_partitions;
        p.num_workers = (int32_t)std::max(1LL, std::min((long long)a.cu_count, items));
        const size_t pl = (size_t)fixed_stream_lds<D>(a.gqa_group);
        return a.k_new ? launch_k(decode_fixed_stream_kernel<D, true>, p, pl, stream)
                       : launch_k(decode_fixed_stream_kernel<D, false>, p, pl, stream);
      }
    }
    return a.k_new ? launch_k(decode_kernel<BF16, D, true, true, false>, a, lds, stream)
                   : launch_k(decode_kernel<BF16, D, true, false, false>, a, lds, stream);
  }
  if (a.scores || a.sink > 0) {  // sink tokens and/or per-head logits (then the column mass)
    hipError_t e = launch_k(decode_kernel<BF16, D, false, false, true>, a, lds, stream);
    if (e != hipSuccess || a.column_mass == nullptr) return e;
    const dim3 grid((a.score_stride + kThreads - 1) / kThreads, a.num_seqs * a.num_kv_heads);
    column_mass_kernel<<<grid, kThreads, 0, stream>>>(a);
    return hipGetLastError();
  }
  return a.k_new ? launch_k(decode_kernel<BF16, D, false, true, false>, a, lds, stream)
                 : launch_k(decode_kernel<BF16, D, false, false, false>, a, lds, stream);
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

#ifndef PKV_ATTN_BODIES_ONLY
hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  if (a.num_seqs <= 0) return hipSuccess;
  return bf16 ? launch_dt<true>(a, head_dim, stream) : launch_dt<false>(a, head_dim, stream);
}
#endif

}  // namespace pkv
