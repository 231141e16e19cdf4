// Check of the caller's side of the paged-cache contract: the device arrays
// every other entry point trusts (block tables, context lengths, the slot
// mapping of an append).
//
// Pages: "Inference Server" (project README mirror), section "The engine" --
// K/V in fixed-size blocks reached through per-sequence block tables, new
// tokens written to the slots the cache manager hands out.  The kernels
// themselves never touch memory outside the pools when these arrays are
// wrong (lengths are clamped, out-of-range block ids and slots skipped); this
// check turns such a caller bug into a reported flag instead of silently
// different attention.
#include "launch.hpp"

namespace pkv {
namespace {

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void check_clear_kernel(uint32_t* flags) {
  if (threadIdx.x == 0) flags[0] = 0u;
}

// One pass over the table entries, one over the slots; each wave ORs its
// findings into the flag word once.  Duplicate slots are found by comparing
// each slot with every later one: O(num_slots^2) reads, a debugging aid.
__global__ __launch_bounds__(kCheckThreads) void check_kernel(CheckArgs a) {
  const long long stride = (long long)gridDim.x * kCheckThreads;
  const long long gid = (long long)blockIdx.x * kCheckThreads + threadIdx.x;
  const long long span = (long long)a.max_blocks_per_seq * 16;
  uint32_t bits = 0;

  const long long entries = (long long)a.num_seqs * a.max_blocks_per_seq;
  for (long long e = gid; e < entries; e += stride) {
    const long long b = e / a.max_blocks_per_seq;
    const long long j = e - b * a.max_blocks_per_seq;
    const int L = a.context_lens[b];
    if (j == 0 && (L < 0 || L > span)) bits |= kCheckBadContextLen;
    const long long Lc = L < 0 ? 0 : (L > span ? span : L);
    if (j * 16 < Lc) {  // an entry the sequence reads
      const int id = a.block_tables[e];
      if (id < 0 || id >= a.num_blocks) bits |= kCheckBadBlockId;
    }
  }

  const long long nslots = (long long)a.num_blocks * 16;
  for (long long i = gid; i < a.num_slots; i += stride) {
    const int s = a.slot_mapping[i];
    if (s < 0) continue;  // a skipped row
    if (s >= nslots) {
      bits |= kCheckBadSlot;
      continue;
    }
    for (long long k = i + 1; k < a.num_slots; ++k) {
      if (a.slot_mapping[k] == s) {
        bits |= kCheckDuplicateSlot;
        break;
      }
    }
  }

#pragma unroll
  for (int off = 32; off > 0; off >>= 1) bits |= (uint32_t)__shfl_xor((int)bits, off);
  if ((threadIdx.x & 63) == 0 && bits != 0u) atomicOr(a.flags, bits);
}

}  // namespace

hipError_t launch_check(const CheckArgs& a, hipStream_t stream) {
  check_clear_kernel<<<1, kCheckThreads, 0, stream>>>(a.flags);
  const long long work = (long long)a.num_seqs * a.max_blocks_per_seq > a.num_slots
                             ? (long long)a.num_seqs * a.max_blocks_per_seq
                             : (long long)a.num_slots;
  long long grid = (work + kCheckThreads - 1) / kCheckThreads;
  if (grid < 1) grid = 1;
  if (grid > 4096) grid = 4096;
  check_kernel<<<(unsigned)grid, kCheckThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pkv
