// Copy-on-write block copy: whole cache blocks duplicated inside the pool.
//
// Pages: "Inference Server" (project README mirror), section "The engine" --
// the KV cache is block-paged with refcounted blocks, so sequences that share
// a prefix share its physical blocks; GitHub README, section "What's inside"
// -- the cache keeps the vLLM/PagedAttention layout.  A sequence about to
// write into a block it shares gets a private copy first; this kernel makes
// those copies, for any number of (source, destination) pairs at once.
//
// In the pool layout one block holds every kv head's K (or V) tile
// contiguously: Hkv * D * 16 elements.  A workgroup copies one pool's block
// of one pair, or a 64 KiB slice of it, with 16-byte loads and stores, eight
// loads in flight per lane.
#include "common.hpp"
#include "launch.hpp"

namespace pkv {
namespace {

// 128 lanes with eight 16-byte loads in flight each, and nontemporal loads
// and stores (the copied blocks are streamed once, not reused through the
// caches): measured 15% faster than 256 lanes with four plain loads each.
constexpr int kCopyThreads = 128;
constexpr int kSliceBytes = 65536;   // bytes per workgroup
constexpr int kUnroll = 8;           // 16-byte loads in flight per lane

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int pair = blockIdx.x;
  const int src = a.src_ids[pair], dst = a.dst_ids[pair];
  if ((unsigned)src >= (unsigned)a.num_blocks || (unsigned)dst >= (unsigned)a.num_blocks ||
      src == dst)
    return;
  char* pool = reinterpret_cast<char*>(blockIdx.y == 0 ? a.k_pool : a.v_pool);
  const size_t bb = a.block_bytes;
  const size_t lo = (size_t)blockIdx.z * kSliceBytes;
  const size_t hi = min(bb, lo + (size_t)kSliceBytes);
  const u32x4* s = reinterpret_cast<const u32x4*>(pool + (size_t)src * bb);
  u32x4* d = reinterpret_cast<u32x4*>(pool + (size_t)dst * bb);
  const size_t n0 = lo / 16, n1 = hi / 16;  // 16-byte units; block bytes are a multiple of 16
  for (size_t i = n0 + threadIdx.x; i < n1; i += (size_t)kCopyThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t k = i + (size_t)u * kCopyThreads;
      if (k < n1) v[u] = __builtin_nontemporal_load(s + k);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t k = i + (size_t)u * kCopyThreads;
      if (k < n1) __builtin_nontemporal_store(v[u], d + k);
    }
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  if (a.num_pairs <= 0) return hipSuccess;
  const dim3 grid(a.num_pairs, 2, (unsigned)((a.block_bytes + kSliceBytes - 1) / kSliceBytes));
  copy_blocks_kernel<<<grid, kCopyThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pkv
