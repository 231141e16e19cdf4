// A mixed batch in one launch: prefill chunks and one-token decode rows.
//
// Pages: "Inference Server" (GitHub README), section "What's inside" --
// chunked prefill, with a mixed batch of prefill chunks and decode steps
// (vLLM-style) left for later because it needs its own attention path;
// "Inference Server -- Architecture Map", section "How a single request
// flows through the system" -- every tick decodes all active requests while
// long prompts are prefilled chunk by chunk.
//
// The grid holds the chunks' prefill workgroups first (the matrix-core
// prefill, one workgroup per (sequence, kv head, 32 positions)), then the
// decode rows' workgroups (the balanced decode split).  Dispatched in grid
// order, the long prefill workgroups start first; the decode workgroups take
// the CUs the prefill leaves free and, as prefill workgroups finish, the rest.
// The decode part is sized to the CUs the prefill leaves free when there are
// any, so that it runs beside the prefill instead of after it.  Both parts
// are the same code as the separate kernels (prefill_mma32_body,
// decode_body), over one dynamic LDS allocation large enough for either.
#define PKV_ATTN_BODIES_ONLY
#include "decode.hip"
#include "prefill.hip"

namespace pkv {
namespace {

template <int D, bool SC, bool FLAT>
__global__ __launch_bounds__(kThreads, 1) void mixed_kernel(PrefillArgs pa, DecodeArgs da) {
  extern __shared__ float lds[];
  if ((int)blockIdx.x < pa.num_items)
    prefill_mma32_body<D, PKV_PREFILL_RING, SC, FLAT>(pa, blockIdx.x, reinterpret_cast<u32x4*>(lds));
  else
    decode_body<true, D, false, false, false>(da, blockIdx.x - pa.num_items, lds);
}

// Decode workgroups beside a prefill of `prefill_wgs` workgroups: the CUs it
// leaves free (at least an eighth of the chip), or the whole chip when it
// fills every CU; at most one per 8 blocks of work and kMaxWorkers.
int mixed_decode_workers(const DecodeArgs& a, int prefill_wgs) {
  long long n = (a.units_bound + PKV_DECODE_MIN_BLOCKS_PER_WG - 1) / PKV_DECODE_MIN_BLOCKS_PER_WG;
  const long long cus = a.cu_count;
  const long long free_cus = prefill_wgs < cus ? std::max(cus - prefill_wgs, (cus + 7) / 8) : cus;
  n = std::min(n, std::min(free_cus, (long long)kMaxWorkers));
  return (int)std::max(n, 1LL);
}

template <int D>
hipError_t launch_m(const PrefillArgs& pa, DecodeArgs da, hipStream_t stream) {
  da.num_workers = mixed_decode_workers(da, pa.num_items);
  // LDS: the prefill's stage ring, or the decode's rings / combine / merge
  size_t lds = kPrefillLdsBytes<D, PKV_PREFILL_RING>;
  lds = std::max(lds, (size_t)kWaves * da.gqa_group * (D + 2) * sizeof(float));
  lds = std::max(lds, (size_t)(4 * kThreads + 2 * 16) * sizeof(float));
  lds = std::max(lds, (size_t)kWaves * kRingBytesPerWave<D>);
  const long long grid = (long long)pa.num_items + da.num_workers;
  if (grid > INT_MAX) return hipErrorInvalidValue;
  const bool flat = prefill_flat<D>(pa);
  auto kernel = pa.softcap > 0.f ? (flat ? mixed_kernel<D, true, true> : mixed_kernel<D, true, false>)
                                 : (flat ? mixed_kernel<D, false, true> : mixed_kernel<D, false, false>);
  hipError_t e = allow_lds(kernel, lds);
  if (e != hipSuccess) return e;
  kernel<<<(unsigned)grid, kThreads, lds, stream>>>(pa, da);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mixed(const PrefillArgs& pa, const DecodeArgs& da, int head_dim,
                        hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_m<64>(pa, da, stream);
    case 128: return launch_m<128>(pa, da, stream);
    case 256: return launch_m<256>(pa, da, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
