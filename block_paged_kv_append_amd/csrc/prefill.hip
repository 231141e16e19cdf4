// Causal chunked prefill over the block-paged cache.
//
// Pages: "Inference Server" (project README mirror), section "The engine" --
// prefill in chunks or batched, paged prefill kernels reading K/V through
// block tables, refcounted shared blocks; "Inference Server -- Architecture
// Map", section "How a single request flows through the system" -- a long
// prompt is prefilled one chunk per tick, after the cached prefix.
//
// Query rows are packed by GQA group: a 16-row matrix-core tile holds
// 16 / G consecutive positions times the G query heads that share one kv
// head, so each K/V block loaded serves G heads at once.  A workgroup is one
// (sequence, kv head, range of positions); each of its four waves owns RT
// row tiles and walks every cache block its rows can see, double-buffered,
// running S^T = K Q^T and P V on the matrix cores with an online softmax per
// row.  Only blocks on the causal diagonal (or at a window edge) are partly
// masked; masking is by select.  Workgroups are numbered so that all ranges
// of one (sequence, kv head) land on the same XCD and share its L2.
#include "attn_tile.hpp"
#include "launch.hpp"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;

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
  if (last_tok < 0) return;
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

template <bool BF16, int D, int RT>
hipError_t launch_p(PrefillArgs a, hipStream_t stream) {
  const int pos_per_item = kWaves * RT * (16 / a.gqa_group);
  // tiles_per_seq was sized by the host for this RT
  if (a.tiles_per_seq * pos_per_item <= 0) return hipErrorInvalidValue;
  prefill_kernel<BF16, D, RT><<<a.num_items, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

// Row tiles per wave: two at head_dim 64/128, one at 256 (register budget).
int prefill_row_tiles(int head_dim) { return head_dim >= 256 ? 1 : 2; }

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  if (a.num_items <= 0) return hipSuccess;
  if (bf16) {
    switch (head_dim) {
      case 64: return launch_p<true, 64, 2>(a, stream);
      case 128: return launch_p<true, 128, 2>(a, stream);
      case 256: return launch_p<true, 256, 1>(a, stream);
    }
  } else {
    switch (head_dim) {
      case 64: return launch_p<false, 64, 2>(a, stream);
      case 128: return launch_p<false, 128, 2>(a, stream);
      case 256: return launch_p<false, 256, 1>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
