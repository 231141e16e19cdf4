// A plain read of a device buffer: the HBM read rate this GPU delivers to a
// kernel that does nothing else, measured beside the attention kernels (the
// decode is judged against HBM read bandwidth; a copy measures reads and
// writes together).  Every lane streams 16-byte loads over a grid-strided
// range, four in flight, and folds them into one word; each workgroup writes
// one word, so the writes are negligible.
#include "common.hpp"
#include "launch.hpp"

namespace pkv {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;

__global__ __launch_bounds__(kReadThreads) void hbm_read_kernel(const u32x4* buf, size_t n16,
                                                                uint32_t* out) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // fold the workgroup's lanes; one word per workgroup
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t part[kReadThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kReadThreads / kWave; ++w) r ^= part[w];
    out[blockIdx.x] = r;
  }
}

// A gather of whole blocks in a given order: block order[i] of two pools
// (block_bytes each, a multiple of 4 KiB), the decode's access pattern (a
// block's K tile and V tile, blocks scattered over the pool).  Workgroup w
// takes entries [w n / N, (w + 1) n / N) of the order, two blocks in flight.
__global__ __launch_bounds__(kReadThreads) void hbm_gather_kernel(const u32x4* k, const u32x4* v,
                                                                  const int32_t* order, int n,
                                                                  int num_blocks, int chunks,
                                                                  uint32_t* out) {
  const int N = gridDim.x, w = blockIdx.x;
  const int i0 = (int)((long long)w * n / N), i1 = (int)((long long)(w + 1) * n / N);
  // an entry outside the buffers reads block 0 instead
  auto blk = [&](int i) -> size_t {
    const int b = order[i];
    return (size_t)((unsigned)b < (unsigned)num_blocks ? b : 0) * chunks;
  };
  auto fold = [](u32x4 x) { return x.x ^ x.y ^ x.z ^ x.w; };
  uint32_t acc = 0;
  for (int i = i0; i < i1; i += 2) {
    const bool two = i + 1 < i1;  // the range's last entry may be alone
    const size_t b0 = blk(i);
    const size_t b1 = blk(two ? i + 1 : i);
    for (int c = threadIdx.x; c < chunks; c += kReadThreads) {
      const u32x4 x0 = __builtin_nontemporal_load(k + b0 + c), y0 = __builtin_nontemporal_load(v + b0 + c);
      const u32x4 x1 = __builtin_nontemporal_load(k + b1 + c), y1 = __builtin_nontemporal_load(v + b1 + c);
      acc ^= fold(x0) ^ fold(y0) ^ (two ? fold(x1) ^ fold(y1) : 0u);
    }
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t part[kReadThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int q = 0; q < kReadThreads / kWave; ++q) r ^= part[q];
    out[w] = r;
  }
}

// Back-to-back 32x32x16 bf16 matrix-core products, one wave per SIMD (a
// workgroup of four waves per CU): the product rate and the shader clock this
// GPU sustains with every matrix core busy, beside the prefill (whose
// throughput is judged against the matrix-core peak).  Four independent
// accumulators, so no product waits for the previous one; lane 0 of each
// workgroup records the shader-clock counter and the constant-rate counter
// before and after the loop.  No memory access inside the loop.
__global__ __launch_bounds__(kReadThreads) void mfma_rate_kernel(unsigned long long* stamps, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (float)i);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  // keeps the products live: the operands are non-negative, so the sum is
  // never -1 and the record always holds the end stamp
  const float sink = c0[0] + c1[1] + c2[2] + c3[3];
  if (threadIdx.x == 0) {
    unsigned long long* s = stamps + (size_t)blockIdx.x * 4;
    s[0] = t0;
    s[1] = t1;
    s[2] = r0;
    s[3] = sink == -1.0f ? 0ull : r1;
  }
}

}  // namespace

hipError_t launch_hbm_gather(const void* k, const void* v, size_t block_bytes, int num_blocks,
                             const int32_t* order, int n, uint32_t* out, int num_wgs,
                             hipStream_t stream) {
  if (n <= 0 || num_wgs <= 0) return hipSuccess;
  hbm_gather_kernel<<<num_wgs, kReadThreads, 0, stream>>>(
      reinterpret_cast<const u32x4*>(k), reinterpret_cast<const u32x4*>(v), order, n, num_blocks,
      (int)(block_bytes / 16), out);
  return hipGetLastError();
}

hipError_t launch_mfma_rate(unsigned long long* stamps, int iters, int num_wgs, hipStream_t stream) {
  if (iters <= 0 || num_wgs <= 0) return hipSuccess;
  mfma_rate_kernel<<<num_wgs, kReadThreads, 0, stream>>>(stamps, iters);
  return hipGetLastError();
}

hipError_t launch_hbm_read(const void* buf, size_t bytes, uint32_t* out, int num_wgs,
                           hipStream_t stream) {
  if (bytes < 16 || num_wgs <= 0) return hipSuccess;
  hbm_read_kernel<<<num_wgs, kReadThreads, 0, stream>>>(reinterpret_cast<const u32x4*>(buf),
                                                        bytes / 16, out);
  return hipGetLastError();
}

}  // namespace pkv
