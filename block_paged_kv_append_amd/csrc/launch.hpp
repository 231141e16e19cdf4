// Internal interface between the C-ABI layer (api.cpp) and the kernel
// translation units.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* slot_mapping;
  void* k_pool;
  void* v_pool;
  int32_t num_tokens;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t elem_bytes;  // 2 (bf16) or 4 (fp32)
};

struct CopyBlocksArgs {
  void* k_pool;
  void* v_pool;
  const int32_t* src_ids;
  const int32_t* dst_ids;
  int32_t num_pairs;
  int32_t num_blocks;
  size_t block_bytes;  // one block of one pool: num_kv_heads * head_dim * 16 * element bytes
};

struct DecodeArgs {
  void* out;
  float* lse;  // may be null
  const void* q;
  const void* k_pool;
  const void* v_pool;
  // fused append: the newest token's rows [num_seqs, num_kv_heads, head_dim];
  // null for a plain decode (the pools are then only read)
  const void* k_new;
  const void* v_new;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;  // lengths are clamped to min(this, max_blocks_per_seq * 16)
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t gqa_group;
  int32_t window;
  float scale;
  float softcap;  // <= 0: off
  // workspace views
  float* part_o;      // [num_slots, gqa_group, head_dim]
  float* part_ml;     // [num_slots, gqa_group, 2]  (max logit in log2 units, sum of 2^(s-m))
  int32_t* seg_count; // [num_seqs, num_kv_heads] pieces stored so far (zero between calls)
  // work decomposition
  int32_t cu_count;         // compute units of the device
  long long units_bound;    // upper bound on (sequence, kv head, block) units
  int32_t units32;          // 1: the split's unit (or item) totals fit in 31 bits
  int32_t num_workers;      // grid size (set by launch_decode in balanced mode)
  int32_t part_blocks;      // 0: balanced split of all blocks; > 0: fixed partitions of this many blocks
  int32_t num_partitions;   // fixed partitions per sequence
  // eviction-policy variant (balanced split only): tokens [0, sink) stay
  // visible beside the window; optional per-head logits
  // [num_seqs, num_q_heads, score_stride] (natural log, -inf where not
  // visible) and per-kv-head attention mass [num_seqs, num_kv_heads, score_stride]
  int32_t sink;
  int32_t score_stride;
  float* scores;
  float* column_mass;
  // timeline build (PKV_TIMELINE) only: per-workgroup phase stamps
  // [kTimelineWgs][kTimelineStamps]; null otherwise, and never written
  unsigned long long* timeline;
};

// Timeline build: stamps per workgroup, and workgroups recorded.
constexpr int kTimelineStamps = 32;
constexpr int kTimelineWgs = 4096;

struct PrefillArgs {
  void* out;
  float* lse;  // may be null
  const void* q;
  const int32_t* cu_q_lens;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_q_tokens;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t gqa_group;
  int32_t window;
  float scale;
  float softcap;
  int32_t tiles_per_seq;  // work items per (sequence, kv head)
  int32_t num_items;      // grid size
  // timeline build (PKV_TIMELINE) only: per-workgroup entry and exit stamps
  // [kTimelineWgs][kTimelineStamps]; null otherwise, and never written
  unsigned long long* timeline;
};

// Decode workspace geometry: the per-segment piece counters (fixed size, at
// offset 0), the partial outputs and their (max, sum) pairs, each 256-byte
// aligned.
constexpr int kMaxWorkers = 1024;  // balanced split: at most this many workgroups
constexpr int kMaxSegments = 65536;  // num_seqs * num_kv_heads per decode call
constexpr size_t kCounterBytes = (size_t)kMaxSegments * sizeof(int32_t);
size_t decode_num_slots(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                        int32_t partition_size);
size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t gqa_group,
                              int32_t head_dim, int32_t max_context_len, int32_t partition_size);

// Check of the caller's metadata (pkv_check_paged_metadata): flag bits.
constexpr uint32_t kCheckBadContextLen = 1u;   // a length < 0 or > max_blocks_per_seq * 16
constexpr uint32_t kCheckBadBlockId = 2u;      // a table entry the sequence reads is outside the pool
constexpr uint32_t kCheckBadSlot = 4u;         // a slot >= num_blocks * 16
constexpr uint32_t kCheckDuplicateSlot = 8u;   // two rows share a non-negative slot

struct CheckArgs {
  const int32_t* block_tables;  // may be null when num_seqs == 0
  const int32_t* context_lens;
  const int32_t* slot_mapping;  // may be null when num_slots == 0
  int32_t num_seqs;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t num_slots;
  uint32_t* flags;  // one word, cleared, then ORed
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
// a plain read of bytes (a multiple of 16) at buf by num_wgs workgroups;
// out [num_wgs] receives one folded word each
hipError_t launch_hbm_read(const void* buf, size_t bytes, uint32_t* out, int num_wgs,
                           hipStream_t stream);
// back-to-back 32x32x16 bf16 products, four waves per workgroup; stamps[4 w .. 4 w + 3]
hipError_t launch_mfma_rate(unsigned long long* stamps, int iters, int num_wgs, hipStream_t stream);
// a gather of whole blocks order[0..n) of two pools of num_blocks blocks
// (block_bytes each, a multiple of 4096; entries outside read block 0)
hipError_t launch_hbm_gather(const void* k, const void* v, size_t block_bytes, int num_blocks,
                             const int32_t* order, int n, uint32_t* out, int num_wgs,
                             hipStream_t stream);
hipError_t launch_check(const CheckArgs& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, bool bf16, hipStream_t stream);
// a mixed batch in one launch (bf16): the prefill of pa's chunks, then the
// balanced decode of da's rows (da.num_workers is chosen here)
hipError_t launch_mixed(const PrefillArgs& pa, const DecodeArgs& da, int head_dim,
                        hipStream_t stream);

// Row tiles (of 16 GQA-packed query rows) per wave in the prefill kernel.
int prefill_row_tiles(int head_dim, bool bf16);

// Set the message pkv_last_error returns (on this thread); returns code.
int record_error(int code, const char* fmt, ...);

}  // namespace pkv
