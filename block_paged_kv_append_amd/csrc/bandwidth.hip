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

}  // namespace

hipError_t launch_hbm_read(const void* buf, size_t bytes, uint32_t* out, int num_wgs,
                           hipStream_t stream) {
  if (bytes < 16 || num_wgs <= 0) return hipSuccess;
  hbm_read_kernel<<<num_wgs, kReadThreads, 0, stream>>>(reinterpret_cast<const u32x4*>(buf),
                                                        bytes / 16, out);
  return hipGetLastError();
}

}  // namespace pkv
