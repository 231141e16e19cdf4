// C ABI of libpkv: argument validation, workspace geometry and launches.
// The operations and their conventions are documented in include/pkv.h.
#include "pkv.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

#ifdef PKV_TIMELINE
// timeline build: where the decode kernels write their phase stamps (and the
// prefill its entry and exit stamps)
unsigned long long* g_timeline = nullptr;
#endif

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    default: return 0;
  }
}

bool head_dim_ok(int32_t d) { return d == 64 || d == 128 || d == 256; }

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int cu_count(int* out) {
  static int cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "hipGetDevice");
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *out = cache[dev];
    return PKV_OK;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return from_hip(e, "hipDeviceGetAttribute");
  if (n <= 0) n = 1;
  if (dev >= 0 && dev < 64) cache[dev] = n;
  *out = n;
  return PKV_OK;
}

// Checks shared by the attention entry points.
int check_common(const char* fn, const void* out, const float* lse, const void* q,
                 const void* k_pool, const void* v_pool, int32_t num_blocks,
                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                 int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim, int32_t block_size,
                 float scale, float softcap, int32_t dtype) {
  if (num_seqs < 0) return fail(PKV_EINVAL, "%s: num_seqs %d < 0", fn, num_seqs);
  if (elem_bytes(dtype) == 0) return fail(PKV_EUNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (!head_dim_ok(head_dim))
    return fail(PKV_EUNSUPPORTED, "%s: head_dim %d not in {64, 128, 256}", fn, head_dim);
  if (block_size != PKV_BLOCK_SIZE)
    return fail(PKV_EUNSUPPORTED, "%s: block_size %d, only 16 is supported", fn, block_size);
  if (gqa_group < 1 || gqa_group > 16)
    return fail(PKV_EUNSUPPORTED, "%s: gqa_group %d outside 1..16", fn, gqa_group);
  if (num_kv_heads < 1) return fail(PKV_EINVAL, "%s: num_kv_heads %d < 1", fn, num_kv_heads);
  if (num_blocks < 1) return fail(PKV_EINVAL, "%s: num_blocks %d < 1", fn, num_blocks);
  if (max_blocks_per_seq < 1)
    return fail(PKV_EINVAL, "%s: max_blocks_per_seq %d < 1", fn, max_blocks_per_seq);
  if ((long long)num_blocks * num_kv_heads * head_dim * PKV_BLOCK_SIZE > (1LL << 40))
    return fail(PKV_EINVAL, "%s: pool of %d blocks too large", fn, num_blocks);
  if (max_context_len < 0 || (long long)max_context_len > (long long)max_blocks_per_seq * PKV_BLOCK_SIZE)
    return fail(PKV_EINVAL, "%s: max_context_len %d outside [0, max_blocks_per_seq * 16 = %lld]",
                fn, max_context_len, (long long)max_blocks_per_seq * PKV_BLOCK_SIZE);
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale is not finite", fn);
  if (std::isnan(softcap) || std::isinf(softcap))
    return fail(PKV_EINVAL, "%s: softcap is not finite", fn);
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "%s: null array argument", fn);
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || (lse && !aligned(lse, 4)))
    return fail(PKV_EINVAL, "%s: misaligned pointer (arrays need 16-byte alignment)", fn);
  return PKV_OK;
}

long long max_units_per_seq(int32_t max_context_len, int32_t window, int32_t sink) {
  long long n = (max_context_len + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
  if (window > 0) {
    const long long w = (window + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE + 1 +
                        (sink + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
    if (w < n) n = w;
  }
  return n;
}

// what a decode entry point adds to the plain decode
struct DecodeExtras {
  const void* k_new = nullptr;  // fused append
  const void* v_new = nullptr;
  int32_t sink = 0;             // AttentionSink tokens
  float* scores = nullptr;      // H2O: per-head logits and column mass
  float* column_mass = nullptr;
  int32_t score_stride = 0;
};

int decode_impl(const char* fn, void* out, float* lse, const void* q, const DecodeExtras& x,
                const void* k_pool, const void* v_pool, int32_t num_blocks, const int32_t* block_tables,
                int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                int32_t block_size, float scale, float softcap, int32_t window,
                int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t dtype,
                hipStream_t stream, pkv::DecodeArgs* build_only = nullptr,
                bool check_only = false) {
  int rc = check_common(fn, out, lse, q, k_pool, v_pool, num_blocks, block_tables,
                        max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_kv_heads,
                        gqa_group, head_dim, block_size, scale, softcap, dtype);
  if (rc != PKV_OK) return rc;
  if ((x.k_new == nullptr) != (x.v_new == nullptr))
    return fail(PKV_EINVAL, "%s: k_new and v_new must both be given", fn);
  if (partition_size < 0 || partition_size % PKV_BLOCK_SIZE != 0)
    return fail(PKV_EUNSUPPORTED, "%s: partition_size %d is not a multiple of 16", fn,
                partition_size);
  if (num_seqs == 0) return PKV_OK;
  if ((long long)num_seqs * num_kv_heads > pkv::kMaxSegments)
    return fail(PKV_EUNSUPPORTED, "%s: num_seqs * num_kv_heads = %lld exceeds %d", fn,
                (long long)num_seqs * num_kv_heads, pkv::kMaxSegments);
  if (check_only) return PKV_OK;  // the arguments alone, before any workspace
  const size_t need = pkv::decode_workspace_bytes(num_seqs, num_kv_heads, gqa_group, head_dim,
                                                  max_context_len, partition_size);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
    return fail(PKV_EWORKSPACE, "%s: workspace of %zu bytes at %p; need %zu bytes, 256-aligned",
                fn, workspace_bytes, workspace, need);

  pkv::DecodeArgs a{};
  a.out = out;
  a.lse = lse;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_new = x.k_new;
  a.v_new = x.v_new;
  a.sink = x.sink;
  a.scores = x.scores;
  a.column_mass = x.column_mass;
  a.score_stride = x.score_stride;
#ifdef PKV_TIMELINE
  a.timeline = g_timeline;
#endif
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.gqa_group = gqa_group;
  a.window = window > 0 ? window : 0;
  a.scale = scale;
  a.softcap = softcap > 0.f ? softcap : 0.f;

  const size_t slots =
      pkv::decode_num_slots(num_seqs, num_kv_heads, max_context_len, partition_size);
  // counters first, at a fixed offset and capacity: whatever sizes a call
  // uses, no other call's data ever lands on them
  char* base = static_cast<char*>(workspace);
  a.seg_count = reinterpret_cast<int32_t*>(base);
  base += pkv::kCounterBytes;
  a.part_o = reinterpret_cast<float*>(base);
  base += align256(slots * gqa_group * head_dim * sizeof(float));
  a.part_ml = reinterpret_cast<float*>(base);

  int cus = 0;
  rc = cu_count(&cus);
  if (rc != PKV_OK) return rc;
  a.cu_count = cus;
  if (partition_size > 0) {
    const int np = (max_context_len + partition_size - 1) / partition_size;
    const long long grid = (long long)num_seqs * num_kv_heads * (np > 0 ? np : 1);
    if (grid > INT_MAX) return fail(PKV_EINVAL, "%s: %lld partitions exceed the grid limit", fn, grid);
    a.part_blocks = partition_size / PKV_BLOCK_SIZE;
    a.num_partitions = np > 0 ? np : 1;
    a.num_workers = (int32_t)grid;
    a.units32 = grid < (1LL << 31) ? 1 : 0;
  } else {
    a.units_bound =
        (long long)num_seqs * num_kv_heads * max_units_per_seq(max_context_len, window, x.sink);
    // the split adds at most 64 cost units per segment
    a.units32 = a.units_bound + (long long)num_seqs * num_kv_heads * 64 < (1LL << 31) ? 1 : 0;
    a.part_blocks = 0;
    a.num_partitions = 0;
    a.num_workers = 0;  // chosen by launch_decode for the kernel variant
  }
  if (build_only) {
    *build_only = a;
    return PKV_OK;
  }
  return from_hip(pkv::launch_decode(a, head_dim, dtype == PKV_BF16, stream), fn);
}

}  // namespace

namespace pkv {

size_t decode_num_slots(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                        int32_t partition_size) {
  if (partition_size == 0) return 2 * (size_t)kMaxWorkers;
  const long long np = (max_context_len + partition_size - 1) / partition_size;
  return (size_t)num_seqs * num_kv_heads * (size_t)(np > 0 ? np : 1);
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                              int32_t head_dim, int32_t max_context_len, int32_t partition_size) {
  const size_t slots = decode_num_slots(num_seqs, num_kv_heads, max_context_len, partition_size);
  return kCounterBytes + align256(slots * gqa_group * head_dim * sizeof(float)) +
         align256(slots * gqa_group * 2 * sizeof(float));
}

int record_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace pkv

namespace {

// ---------------------------------------------------------------------------
// Scratch of the allocation-free decode (paged_attn_decode_no_alloc): the
// decode workspace (segment counters, then the partial results) as a static
// device array, one copy per GPU, held until the process ends.  Its size is
// the largest balanced-split workspace (group 16, head_dim 256): 32.5 MiB.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): the first call on each device looks up
// the device address once and keeps it.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes =
    pkv::kCounterBytes + ((2 * (size_t)pkv::kMaxWorkers * 16 * 256 * sizeof(float) + 255) & ~size_t(255)) +
    ((2 * (size_t)pkv::kMaxWorkers * 16 * 2 * sizeof(float) + 255) & ~size_t(255));

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The current device's scratch address; the first call on a device looks it
// up and clears the counters (a kernel on `stream`, so that a call made
// under graph capture records it instead of running it).
int device_scratch(const char* fn, hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_EUNSUPPORTED, "%s: device %d", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return from_hip(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    const int words = (int)(pkv::kCounterBytes / sizeof(uint32_t));
    zero_words_kernel<<<(words + 255) / 256, 256, 0, stream>>>(static_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return from_hip(e, "clearing the scratch counters");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_err; }

#ifdef PKV_TIMELINE
// Timeline build only (not declared in pkv.h): the device buffer of
// kTimelineWgs x kTimelineStamps words the next decode launches stamp (NULL:
// none), and the stamp clock's rate in kHz.
void pkv_timeline_set(unsigned long long* buf) { g_timeline = buf; }
int pkv_timeline_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}
#endif

int paged_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                    int32_t num_tokens, void* k_pool, void* v_pool, int32_t num_blocks,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                    struct ihipStream_t* stream) {
  const char* fn = "paged_kv_append";
  if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens %d < 0", fn, num_tokens);
  const int es = elem_bytes(dtype);
  if (es == 0) return fail(PKV_EUNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (!head_dim_ok(head_dim))
    return fail(PKV_EUNSUPPORTED, "%s: head_dim %d not in {64, 128, 256}", fn, head_dim);
  if (block_size != PKV_BLOCK_SIZE)
    return fail(PKV_EUNSUPPORTED, "%s: block_size %d, only 16 is supported", fn, block_size);
  if (num_kv_heads < 1) return fail(PKV_EINVAL, "%s: num_kv_heads %d < 1", fn, num_kv_heads);
  if (num_blocks < 1) return fail(PKV_EINVAL, "%s: num_blocks %d < 1", fn, num_blocks);
  if ((long long)num_blocks * PKV_BLOCK_SIZE > INT_MAX)
    return fail(PKV_EINVAL, "%s: %d blocks overflow the int32 slot range", fn, num_blocks);
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_pool || !v_pool)
    return fail(PKV_EINVAL, "%s: null array argument", fn);
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(slot_mapping, 4))
    return fail(PKV_EINVAL, "%s: misaligned pointer (arrays need 16-byte alignment)", fn);
  pkv::AppendArgs a{k_new, v_new, slot_mapping, k_pool, v_pool, num_tokens, num_blocks,
                    num_kv_heads, head_dim, es};
  return from_hip(pkv::launch_append(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

int paged_kv_copy_blocks(void* k_pool, void* v_pool, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, const int32_t* src_ids,
                         const int32_t* dst_ids, int32_t num_pairs, int32_t dtype,
                         struct ihipStream_t* stream) {
  const char* fn = "paged_kv_copy_blocks";
  const int es = elem_bytes(dtype);
  if (es == 0) return fail(PKV_EUNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (block_size != PKV_BLOCK_SIZE)
    return fail(PKV_EUNSUPPORTED, "%s: block_size %d (only 16)", fn, block_size);
  if (!head_dim_ok(head_dim)) return fail(PKV_EUNSUPPORTED, "%s: head_dim %d", fn, head_dim);
  if (num_pairs < 0 || num_blocks < 0 || num_kv_heads < 1)
    return fail(PKV_EINVAL, "%s: num_pairs %d, num_blocks %d, num_kv_heads %d", fn, num_pairs,
                num_blocks, num_kv_heads);
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src_ids || !dst_ids)
    return fail(PKV_EINVAL, "%s: null pointer", fn);
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(src_ids, 4) || !aligned(dst_ids, 4))
    return fail(PKV_EINVAL, "%s: misaligned pointer", fn);
  pkv::CopyBlocksArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.src_ids = src_ids;
  a.dst_ids = dst_ids;
  a.num_pairs = num_pairs;
  a.num_blocks = num_blocks;
  a.block_bytes = (size_t)num_kv_heads * head_dim * PKV_BLOCK_SIZE * es;
  return from_hip(pkv::launch_copy_blocks(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

int pkv_hbm_read_probe(const void* buf, size_t bytes, uint32_t* out, int32_t num_wgs,
                       struct ihipStream_t* stream) {
  const char* fn = "pkv_hbm_read_probe";
  if (bytes == 0) return PKV_OK;
  if (buf == nullptr || out == nullptr) return fail(PKV_EINVAL, "%s: null pointer", fn);
  if (bytes % 16 != 0 || !aligned(buf, 16) || !aligned(out, 4))
    return fail(PKV_EINVAL, "%s: bytes %zu not a multiple of 16, or misaligned pointers", fn,
                bytes);
  if (num_wgs < 1 || num_wgs > (1 << 20)) return fail(PKV_EINVAL, "%s: num_wgs %d", fn, num_wgs);
  return from_hip(pkv::launch_hbm_read(buf, bytes, out, num_wgs,
                                       reinterpret_cast<hipStream_t>(stream)), fn);
}

int pkv_mfma_rate_probe(unsigned long long* stamps, int32_t iters, int32_t num_wgs,
                        struct ihipStream_t* stream) {
  const char* fn = "pkv_mfma_rate_probe";
  if (stamps == nullptr || !aligned(stamps, 8)) return fail(PKV_EINVAL, "%s: stamps null or misaligned", fn);
  if (iters < 1 || iters > (1 << 24)) return fail(PKV_EINVAL, "%s: iters %d", fn, iters);
  if (num_wgs < 1 || num_wgs > (1 << 20)) return fail(PKV_EINVAL, "%s: num_wgs %d", fn, num_wgs);
  return from_hip(pkv::launch_mfma_rate(stamps, iters, num_wgs, reinterpret_cast<hipStream_t>(stream)),
                  fn);
}

int pkv_hbm_gather_probe(const void* k, const void* v, size_t block_bytes, int32_t num_blocks,
                         const int32_t* order, int32_t n, uint32_t* out, int32_t num_wgs,
                         struct ihipStream_t* stream) {
  const char* fn = "pkv_hbm_gather_probe";
  if (n == 0) return PKV_OK;
  if (!k || !v || !order || !out) return fail(PKV_EINVAL, "%s: null pointer", fn);
  if (n < 0 || num_blocks < 1 || block_bytes == 0 || block_bytes % 4096 != 0 ||
      block_bytes / 16 > (size_t)INT_MAX || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(order, 4) || !aligned(out, 4))
    return fail(PKV_EINVAL, "%s: n %d, block_bytes %zu (a multiple of 4096), or misaligned", fn,
                n, block_bytes);
  if (num_wgs < 1 || num_wgs > (1 << 20)) return fail(PKV_EINVAL, "%s: num_wgs %d", fn, num_wgs);
  return from_hip(pkv::launch_hbm_gather(k, v, block_bytes, num_blocks, order, n, out, num_wgs,
                                         reinterpret_cast<hipStream_t>(stream)), fn);
}

int pkv_check_paged_metadata(const int32_t* block_tables, const int32_t* context_lens,
                             int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                             const int32_t* slot_mapping, int32_t num_slots, uint32_t* flags,
                             struct ihipStream_t* stream) {
  const char* fn = "pkv_check_paged_metadata";
  if (num_seqs < 0 || num_slots < 0)
    return fail(PKV_EINVAL, "%s: num_seqs %d, num_slots %d", fn, num_seqs, num_slots);
  if (max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(PKV_EINVAL, "%s: max_blocks_per_seq %d, num_blocks %d", fn, max_blocks_per_seq,
                num_blocks);
  if ((long long)num_blocks * PKV_BLOCK_SIZE > INT_MAX)
    return fail(PKV_EINVAL, "%s: %d blocks overflow the int32 slot range", fn, num_blocks);
  if (flags == nullptr) return fail(PKV_EINVAL, "%s: null flags", fn);
  if (num_seqs > 0 && (block_tables == nullptr || context_lens == nullptr))
    return fail(PKV_EINVAL, "%s: null block_tables or context_lens", fn);
  if (num_slots > 0 && slot_mapping == nullptr) return fail(PKV_EINVAL, "%s: null slot_mapping", fn);
  if (!aligned(flags, 4) || !aligned(block_tables, 4) || !aligned(context_lens, 4) ||
      !aligned(slot_mapping, 4))
    return fail(PKV_EINVAL, "%s: misaligned pointer", fn);
  pkv::CheckArgs a{block_tables, context_lens, slot_mapping, num_seqs, max_blocks_per_seq,
                   num_blocks, num_slots, flags};
  return from_hip(pkv::launch_check(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_kv_heads,
                                        int32_t gqa_group, int32_t head_dim,
                                        int32_t max_context_len, int32_t partition_size) {
  if (num_seqs < 0 || num_kv_heads < 1 || gqa_group < 1 || gqa_group > 16 ||
      !head_dim_ok(head_dim) || max_context_len < 0 || partition_size < 0 ||
      partition_size % PKV_BLOCK_SIZE != 0)
    return 0;
  return pkv::decode_workspace_bytes(num_seqs, num_kv_heads, gqa_group, head_dim, max_context_len,
                                     partition_size);
}

int paged_attn_decode(void* out, float* lse, const void* q, const void* k_pool,
                      const void* v_pool, int32_t num_blocks, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t max_context_len, int32_t num_seqs, int32_t num_kv_heads,
                      int32_t gqa_group, int32_t head_dim, int32_t block_size, float scale,
                      float softcap, int32_t window, void* workspace, size_t workspace_bytes,
                      int32_t dtype, struct ihipStream_t* stream) {
  return decode_impl("paged_attn_decode", out, lse, q, DecodeExtras{}, k_pool, v_pool,
                     num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_kv_heads,
                     gqa_group, head_dim, block_size, scale, softcap, window, 0, workspace,
                     workspace_bytes, dtype, reinterpret_cast<hipStream_t>(stream));
}

int paged_attn_decode_splitk(void* out, float* lse, const void* q, const void* k_pool,
                             const void* v_pool, int32_t num_blocks,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t max_context_len,
                             int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                             int32_t head_dim, int32_t block_size, float scale, float softcap,
                             int32_t window, int32_t partition_size, void* workspace,
                             size_t workspace_bytes, int32_t dtype, struct ihipStream_t* stream) {
  if (partition_size <= 0 || partition_size % PKV_BLOCK_SIZE != 0)
    return fail(PKV_EUNSUPPORTED, "paged_attn_decode_splitk: partition_size %d is not a positive "
                "multiple of 16", partition_size);
  return decode_impl("paged_attn_decode_splitk", out, lse, q, DecodeExtras{}, k_pool, v_pool,
                     num_blocks,
                     block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                     num_kv_heads, gqa_group, head_dim, block_size, scale, softcap, window,
                     partition_size, workspace, workspace_bytes, dtype,
                     reinterpret_cast<hipStream_t>(stream));
}

int paged_attn_decode_no_alloc(void* out, float* lse, const void* q, const void* k_pool,
                               const void* v_pool, int32_t num_blocks,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t max_context_len,
                               int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                               int32_t head_dim, int32_t block_size, float scale, float softcap,
                               int32_t window, int32_t partition_size, int32_t dtype,
                               struct ihipStream_t* stream) {
  const char* fn = "paged_attn_decode_no_alloc";
  if (partition_size < 0 || partition_size % PKV_BLOCK_SIZE != 0)
    return fail(PKV_EUNSUPPORTED, "%s: partition_size %d is not 0 or a positive multiple of 16",
                fn, partition_size);
  // the same argument checks as the workspace form first, so that a bad call
  // fails for its own reason before the scratch size is considered
  int rc = decode_impl(fn, out, lse, q, DecodeExtras{}, k_pool, v_pool, num_blocks, block_tables,
                       max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_kv_heads,
                       gqa_group, head_dim, block_size, scale, softcap, window, partition_size,
                       nullptr, SIZE_MAX, dtype, reinterpret_cast<hipStream_t>(stream),
                       nullptr, /*check_only=*/true);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  const size_t need = pkv::decode_workspace_bytes(num_seqs, num_kv_heads, gqa_group, head_dim,
                                                  max_context_len, partition_size);
  if (need > kNoAllocScratchBytes)
    return fail(PKV_EWORKSPACE,
                "%s: these sizes need %zu bytes of scratch; the static scratch holds %zu (use "
                "paged_attn_decode_splitk with a workspace, or a larger partition_size)",
                fn, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  rc = device_scratch(fn, reinterpret_cast<hipStream_t>(stream), &ws);
  if (rc != PKV_OK) return rc;
  return decode_impl(fn, out, lse, q, DecodeExtras{}, k_pool, v_pool, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_kv_heads,
                     gqa_group, head_dim, block_size, scale, softcap, window, partition_size, ws,
                     kNoAllocScratchBytes, dtype, reinterpret_cast<hipStream_t>(stream));
}

int paged_attn_decode_append(void* out, float* lse, const void* q, const void* k_new,
                             const void* v_new, void* k_pool, void* v_pool, int32_t num_blocks,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t max_context_len,
                             int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                             int32_t head_dim, int32_t block_size, float scale, float softcap,
                             int32_t window, int32_t partition_size, void* workspace,
                             size_t workspace_bytes, int32_t dtype, struct ihipStream_t* stream) {
  const char* fn = "paged_attn_decode_append";
  if (k_new == nullptr || v_new == nullptr)
    return fail(PKV_EINVAL, "%s: k_new and v_new are required", fn);
  if (num_seqs > 0 && (!aligned(k_new, 16) || !aligned(v_new, 16)))
    return fail(PKV_EINVAL, "%s: k_new / v_new must be 16-byte aligned", fn);
  DecodeExtras x;
  x.k_new = k_new;
  x.v_new = v_new;
  return decode_impl(fn, out, lse, q, x, k_pool, v_pool, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_kv_heads,
                     gqa_group, head_dim, block_size, scale, softcap, window, partition_size,
                     workspace, workspace_bytes, dtype, reinterpret_cast<hipStream_t>(stream));
}

int paged_attn_decode_sink_h2o(void* out, float* lse, const void* q, const void* k_pool,
                               const void* v_pool, int32_t num_blocks, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t max_context_len, int32_t num_seqs, int32_t num_kv_heads,
                               int32_t gqa_group, int32_t head_dim, int32_t block_size,
                               float scale, float softcap, int32_t window, int32_t sink_tokens,
                               float* scores, float* column_mass, int32_t score_stride,
                               void* workspace, size_t workspace_bytes, int32_t dtype,
                               struct ihipStream_t* stream) {
  const char* fn = "paged_attn_decode_sink_h2o";
  if (sink_tokens < 0) return fail(PKV_EINVAL, "%s: sink_tokens %d", fn, sink_tokens);
  if ((scores == nullptr) != (column_mass == nullptr))
    return fail(PKV_EINVAL, "%s: scores and column_mass go together", fn);
  if (column_mass != nullptr) {
    if (lse == nullptr) return fail(PKV_EINVAL, "%s: column_mass needs lse", fn);
    if (score_stride < max_context_len || score_stride % PKV_BLOCK_SIZE != 0)
      return fail(PKV_EINVAL, "%s: score_stride %d: a multiple of 16 >= max_context_len %d", fn,
                  score_stride, max_context_len);
    if (!aligned(scores, 16) || !aligned(column_mass, 4))
      return fail(PKV_EINVAL, "%s: scores must be 16-byte aligned, column_mass 4-byte", fn);
  }
  DecodeExtras x;
  x.sink = window > 0 ? sink_tokens : 0;
  x.scores = scores;
  x.column_mass = column_mass;
  x.score_stride = column_mass != nullptr ? score_stride : 0;
  return decode_impl(fn, out, lse, q, x, k_pool, v_pool, num_blocks, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_kv_heads,
                     gqa_group, head_dim, block_size, scale, softcap, window, 0, workspace,
                     workspace_bytes, dtype, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

// Checks a prefill call and fills its kernel arguments; *empty is set when
// there is nothing to compute (the call is then a no-op).
int prefill_build(const char* fn, void* out, float* lse, const void* q, const int32_t* cu_q_lens,
                  int32_t num_q_tokens, int32_t max_q_len, const void* k_pool, const void* v_pool,
                  int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                  int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim, int32_t block_size,
                  float scale, float softcap, int32_t window, int32_t dtype, pkv::PrefillArgs* out_a,
                  bool* empty) {
  *empty = true;
  int rc = check_common(fn, out, lse, q, k_pool, v_pool, num_blocks, block_tables,
                        max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_kv_heads,
                        gqa_group, head_dim, block_size, scale, softcap, dtype);
  if (rc != PKV_OK) return rc;
  if (16 % gqa_group != 0)
    return fail(PKV_EUNSUPPORTED, "%s: gqa_group %d must divide 16", fn, gqa_group);
  if (num_q_tokens < 0 || max_q_len < 0)
    return fail(PKV_EINVAL, "%s: num_q_tokens %d / max_q_len %d < 0", fn, num_q_tokens, max_q_len);
  if (max_q_len > max_context_len)
    return fail(PKV_EINVAL, "%s: max_q_len %d > max_context_len %d", fn, max_q_len,
                max_context_len);
  if (num_seqs == 0 || num_q_tokens == 0 || max_q_len == 0) return PKV_OK;
  if (!cu_q_lens || !aligned(cu_q_lens, 4))
    return fail(PKV_EINVAL, "%s: cu_q_lens null or misaligned", fn);

  pkv::PrefillArgs& a = *out_a;
  a = pkv::PrefillArgs{};
  a.out = out;
  a.lse = lse;
  a.q = q;
  a.cu_q_lens = cu_q_lens;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_q_tokens = num_q_tokens;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.gqa_group = gqa_group;
  a.window = window > 0 ? window : 0;
  a.scale = scale;
  a.softcap = softcap > 0.f ? softcap : 0.f;
  const int per_item = 4 * pkv::prefill_row_tiles(head_dim, dtype == PKV_BF16) * (16 / gqa_group);
  a.tiles_per_seq = (max_q_len + per_item - 1) / per_item;
  const long long items = (long long)num_seqs * num_kv_heads * a.tiles_per_seq;
  if (items > INT_MAX) return fail(PKV_EINVAL, "%s: %lld work items exceed the grid limit", fn, items);
  a.num_items = (int32_t)items;
#ifdef PKV_TIMELINE
  a.timeline = g_timeline;
#endif
  *empty = false;
  return PKV_OK;
}

extern "C" {

int paged_attn_prefill(void* out, float* lse, const void* q, const int32_t* cu_q_lens,
                       int32_t num_q_tokens, int32_t max_q_len, const void* k_pool,
                       const void* v_pool, int32_t num_blocks, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t max_context_len, int32_t num_seqs, int32_t num_kv_heads,
                       int32_t gqa_group, int32_t head_dim, int32_t block_size, float scale,
                       float softcap, int32_t window, int32_t dtype, struct ihipStream_t* stream) {
  const char* fn = "paged_attn_prefill";
  pkv::PrefillArgs a;
  bool empty = true;
  const int rc = prefill_build(fn, out, lse, q, cu_q_lens, num_q_tokens, max_q_len, k_pool, v_pool,
                               num_blocks, block_tables, max_blocks_per_seq, context_lens,
                               max_context_len, num_seqs, num_kv_heads, gqa_group, head_dim,
                               block_size, scale, softcap, window, dtype, &a, &empty);
  if (rc != PKV_OK || empty) return rc;
  return from_hip(pkv::launch_prefill(a, head_dim, dtype == PKV_BF16,
                                      reinterpret_cast<hipStream_t>(stream)),
                  fn);
}

int paged_attn_mixed(void* out, float* lse, const void* q, const int32_t* cu_q_lens,
                     int32_t num_prefill_seqs, int32_t num_prefill_tokens, int32_t max_q_len,
                     const void* k_pool, const void* v_pool, int32_t num_blocks,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                     int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                     int32_t block_size, float scale, float softcap, int32_t window,
                     void* workspace, size_t workspace_bytes, int32_t dtype,
                     struct ihipStream_t* stream) {
  const char* fn = "paged_attn_mixed";
  if (num_prefill_seqs < 0 || num_prefill_seqs > num_seqs || num_prefill_tokens < 0 ||
      (num_prefill_seqs == 0) != (num_prefill_tokens == 0))
    return fail(PKV_EINVAL, "%s: %d prefill sequences / %d prefill rows of %d sequences", fn,
                num_prefill_seqs, num_prefill_tokens, num_seqs);
  const int es = elem_bytes(dtype);
  if (es == 0) return fail(PKV_EUNSUPPORTED, "%s: dtype %d", fn, dtype);
  const int32_t P = num_prefill_seqs, Bd = num_seqs - num_prefill_seqs;
  const size_t row = (size_t)num_kv_heads * gqa_group * head_dim * es;  // one q / out row
  int rc = PKV_OK;
  char* o = static_cast<char*>(out) + (size_t)num_prefill_tokens * row;
  const char* qd = static_cast<const char*>(q) + (size_t)num_prefill_tokens * row;
  float* ld = lse ? lse + (size_t)num_prefill_tokens * num_kv_heads * gqa_group : nullptr;
  if (P > 0 && Bd > 0 && dtype == PKV_BF16) {
    // both parts in one launch
    pkv::PrefillArgs pa;
    bool empty = true;
    rc = prefill_build(fn, out, lse, q, cu_q_lens, num_prefill_tokens, max_q_len, k_pool, v_pool,
                       num_blocks, block_tables, max_blocks_per_seq, context_lens,
                       max_context_len, P, num_kv_heads, gqa_group, head_dim, block_size, scale,
                       softcap, window, dtype, &pa, &empty);
    if (rc != PKV_OK) return rc;
    pkv::DecodeArgs da;
    rc = decode_impl(fn, o, ld, qd, DecodeExtras{}, k_pool, v_pool, num_blocks,
                     block_tables + (size_t)P * max_blocks_per_seq, max_blocks_per_seq,
                     context_lens + P, max_context_len, Bd, num_kv_heads, gqa_group, head_dim,
                     block_size, scale, softcap, window, 0, workspace, workspace_bytes, dtype,
                     reinterpret_cast<hipStream_t>(stream), &da);
    if (rc != PKV_OK) return rc;
    if (!empty)
      return from_hip(pkv::launch_mixed(pa, da, head_dim, reinterpret_cast<hipStream_t>(stream)),
                      fn);
    return from_hip(pkv::launch_decode(da, head_dim, true, reinterpret_cast<hipStream_t>(stream)),
                    fn);
  }
  if (P > 0) {
    rc = paged_attn_prefill(out, lse, q, cu_q_lens, num_prefill_tokens, max_q_len, k_pool, v_pool,
                            num_blocks, block_tables, max_blocks_per_seq, context_lens,
                            max_context_len, P, num_kv_heads, gqa_group, head_dim, block_size,
                            scale, softcap, window, dtype, stream);
    if (rc != PKV_OK) return rc;
  }
  if (Bd > 0) {
    rc = decode_impl(fn, o, ld, qd, DecodeExtras{}, k_pool, v_pool, num_blocks,
                     block_tables + (size_t)P * max_blocks_per_seq, max_blocks_per_seq,
                     context_lens + P, max_context_len, Bd, num_kv_heads, gqa_group, head_dim,
                     block_size, scale, softcap, window, 0, workspace, workspace_bytes, dtype,
                     reinterpret_cast<hipStream_t>(stream));
  }
  return rc;
}

}  // extern "C"
