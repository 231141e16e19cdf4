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
// piece that is a whole segment writes the output directly.  Otherwise it
// stores (max, sum, unnormalised output) to the workspace and adds its block
// count to the segment's counter; the workgroup that completes the count
// merges all pieces of the segment by log-sum-exp, writes the output and
// resets the counter to zero for the next call.
//
// Inner loop per wave: double-buffered block loads (K and V fragments for
// the next block are in flight while the current block is computed), S^T =
// K Q^T on the matrix cores with the GQA group's query heads as the 16
// columns (padded with zero rows), mask by select, online softmax in base 2
// with cross-lane max over the 4 lanes that share a head, then P V on the
// matrix cores.
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

// Merge the partials of segment (b, g) listed by `slots`, then write the
// output.  Called by every thread of the completing workgroup.
template <bool BF16, int D, typename SlotList>
__device__ void merge_segment(const DecodeArgs& a, int b, int g, SlotList slots) {
  const int G = a.gqa_group;
  const int nvec = G * D / 4;
  for (int e = threadIdx.x; e < nvec; e += kThreads) {
    const int h = (e * 4) / D, d = (e * 4) % D;
    float M = kNegInf, L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    slots.for_each([&](int slot) {
      const float mk = a.part_ml[((size_t)slot * G + h) * 2];
      const float lk = a.part_ml[((size_t)slot * G + h) * 2 + 1];
      if (!(lk > 0.f)) return;
      const f32x4 ok = *reinterpret_cast<const f32x4*>(a.part_o + ((size_t)slot * G + h) * D + d);
      const float Mn = fmaxf(M, mk);
      const float sa = fast_exp2(M - Mn);  // 0 when M = -inf
      const float sb = fast_exp2(mk - Mn);
      O = O * sa + ok * sb;
      L = L * sa + lk * sb;
      M = Mn;
    });
    finalize_vec<BF16, D>(a, b, g * G + h, d, O, L, M);
  }
}

struct SplitSlots {  // fixed partitions p_lo .. p_hi of one segment
  int base, p_lo, p_hi;
  template <typename F>
  __device__ void for_each(F&& f) const {
    for (int p = p_lo; p <= p_hi; ++p) f(base + p);
  }
};

struct BalancedSlots {  // workgroups whose ranges meet [S, E)
  long long W, S, E;
  int N;
  template <typename F>
  __device__ void for_each(F&& f) const {
    const int w_first = (int)(((S + 1) * N - 1) / W);
    const int w_last = (int)((E * N - 1) / W);
    for (int w = w_first; w <= w_last; ++w) {
      const long long a0 = (long long)w * W / N, a1 = (long long)(w + 1) * W / N;
      if (a0 == a1) continue;  // empty range: wrote nothing
      f(a0 < S ? 2 * w + 1 : 2 * w);
    }
  }
};

// One piece: all four waves of the workgroup.
template <bool BF16, int D, typename SlotList>
__device__ void run_piece(const DecodeArgs& a, const LogitXform& xf, const Piece& pc,
                          SlotList slots, float* lds, int* flag) {
  using T = typename Elem<BF16>::T;
  using KV = KVFrag<BF16, D>;
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

  auto fetch = [&](KV& buf, int jl) -> bool {
    const int phys = bt[jl];
    if ((unsigned)phys >= (unsigned)a.num_blocks) {
      buf.zero();
      return false;
    }
    const size_t off = ((size_t)phys * Hkv + g) * kTile;
    buf.load(kpool + off, vpool + off, lane);
    return true;
  };

  auto step = [&](KV& buf, bool ok, int jl) {
    const int tok0 = (sp.first_blk + jl) * kBlock;
    const f32x4 sc = qk_tile<D>(buf, qf);
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
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s2[r] - m_use);
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
    // O rows are heads 4j + r: fetch their rescale factors from lanes 4j + r
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
    if (ok && tok0 + kBlock > sp.L) buf.mask_v_tail(sp.L - tok0, lane);
    pv_tile<D>(o, p, buf);
  };

  // double-buffered walk over this wave's blocks j0 + wave, j0 + wave + 4, ...
  KV bufA, bufB;
  bool okA = false, okB = false;
  int jl = pc.j0 + wave;
  if (jl < pc.j1) okA = fetch(bufA, jl);
  while (jl < pc.j1) {
    int jn = jl + kWaves;
    if (jn < pc.j1) okB = fetch(bufB, jn);
    step(bufA, okA, jl);
    jl = jn;
    if (jl >= pc.j1) break;
    jn = jl + kWaves;
    if (jn < pc.j1) okA = fetch(bufA, jn);
    step(bufB, okB, jl);
    jl = jn;
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

  if (!whole) {
    __threadfence();  // publish this piece before counting it
    __syncthreads();
    int* counter = a.counters + (size_t)b * Hkv + g;
    if (threadIdx.x == 0) {
      const int add = pc.j1 - pc.j0;
      const int old = atomicAdd(counter, add);
      *flag = (old + add == sp.nb);
    }
    __syncthreads();
    if (*flag) {
      __threadfence();  // see every other piece of the segment
      merge_segment<BF16, D>(a, b, g, slots);
      if (threadIdx.x == 0) atomicExch(counter, 0);
    }
  }
  __syncthreads();  // LDS is reused by the next piece
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

template <bool BF16, int D, bool FIXED>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeArgs a) {
  extern __shared__ float lds[];
  __shared__ int flag;
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
    const SplitSlots slots{seg * NP, pc.sp.first_blk / PB, last_blk / PB};
    run_piece<BF16, D>(a, xf, pc, slots, lds, &flag);
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
      const BalancedSlots slots{W, pc.S, E, N};
      run_piece<BF16, D>(a, xf, pc, slots, lds, &flag);
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

// The combine buffer holds the four waves' partial outputs: up to 66 KiB for
// a group of 16 at head_dim 256, above the default 64 KiB dynamic-LDS limit.
template <typename K>
hipError_t allow_lds(K kernel, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <bool BF16, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)kWaves * a.gqa_group * (D + 2) * sizeof(float);
  hipError_t e;
  if (a.part_blocks > 0) {
    if ((e = allow_lds(decode_kernel<BF16, D, true>, lds)) != hipSuccess) return e;
    decode_kernel<BF16, D, true><<<a.num_workers, kThreads, lds, stream>>>(a);
  } else {
    if ((e = allow_lds(decode_kernel<BF16, D, false>, lds)) != hipSuccess) return e;
    decode_kernel<BF16, D, false><<<a.num_workers, kThreads, lds, stream>>>(a);
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
  if (a.num_seqs <= 0 || a.num_workers <= 0) return hipSuccess;
  return bf16 ? launch_dt<true>(a, head_dim, stream) : launch_dt<false>(a, head_dim, stream);
}

}  // namespace pkv
