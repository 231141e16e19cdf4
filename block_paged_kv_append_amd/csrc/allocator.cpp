// Refcounted block allocator with copy-on-write, feeding the block tables.
//
// Pages: "Inference Server" (project README mirror), section "The engine" --
// the KV cache is block-paged with refcounted blocks; sequences that share a
// prefix hold the same physical blocks.  The allocator hands out block ids,
// counts how many tables hold each block, and, before a sequence writes into
// a block that others also hold, swaps in a private block and reports the
// (source, destination) pair that paged_kv_copy_blocks must copy.
//
// Host-only bookkeeping (no HIP calls); one mutex per allocator.
#include <mutex>
#include <new>
#include <vector>

#include "launch.hpp"
#include "pkv.h"

using pkv::record_error;

struct pkv_block_allocator {
  std::mutex mu;
  std::vector<int32_t> refs;   // refcount per block (0 = free)
  std::vector<int32_t> free;   // free ids, next one to hand out at the back
};

namespace {

bool valid(const pkv_block_allocator* a, int32_t id) {
  return id >= 0 && (size_t)id < a->refs.size();
}

}  // namespace

extern "C" {

int pkv_allocator_create(pkv_block_allocator** out, int32_t num_blocks) {
  if (out == nullptr) return record_error(PKV_EINVAL, "pkv_allocator_create: out is null");
  *out = nullptr;
  if (num_blocks < 0)
    return record_error(PKV_EINVAL, "pkv_allocator_create: num_blocks %d", num_blocks);
  pkv_block_allocator* a = new (std::nothrow) pkv_block_allocator();
  if (a == nullptr) return record_error(PKV_ENOMEM, "pkv_allocator_create: out of host memory");
  try {
    a->refs.assign((size_t)num_blocks, 0);
    a->free.reserve((size_t)num_blocks);
    for (int32_t i = num_blocks - 1; i >= 0; --i) a->free.push_back(i);  // hands out 0, 1, 2, ...
  } catch (...) {
    delete a;
    return record_error(PKV_ENOMEM, "pkv_allocator_create: out of host memory");
  }
  *out = a;
  return PKV_OK;
}

void pkv_allocator_destroy(pkv_block_allocator* a) { delete a; }

int32_t pkv_allocator_num_free(pkv_block_allocator* a) {
  if (a == nullptr) return -1;
  std::lock_guard<std::mutex> lock(a->mu);
  return (int32_t)a->free.size();
}

int32_t pkv_allocator_refcount(pkv_block_allocator* a, int32_t block) {
  if (a == nullptr) return -1;
  std::lock_guard<std::mutex> lock(a->mu);
  return valid(a, block) ? a->refs[(size_t)block] : -1;
}

int pkv_allocator_alloc(pkv_block_allocator* a, int32_t n, int32_t* ids) {
  const char* fn = "pkv_allocator_alloc";
  if (a == nullptr || (n > 0 && ids == nullptr) || n < 0)
    return record_error(PKV_EINVAL, "%s: null allocator/ids or n = %d", fn, n);
  std::lock_guard<std::mutex> lock(a->mu);
  if ((size_t)n > a->free.size())
    return record_error(PKV_ENOMEM, "%s: %d blocks asked, %zu free", fn, n, a->free.size());
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = a->free.back();
    a->free.pop_back();
    a->refs[(size_t)id] = 1;
    ids[i] = id;
  }
  return PKV_OK;
}

int pkv_allocator_share(pkv_block_allocator* a, const int32_t* ids, int32_t n) {
  const char* fn = "pkv_allocator_share";
  if (a == nullptr || (n > 0 && ids == nullptr) || n < 0)
    return record_error(PKV_EINVAL, "%s: null allocator/ids or n = %d", fn, n);
  std::lock_guard<std::mutex> lock(a->mu);
  for (int32_t i = 0; i < n; ++i)  // check all first: all or nothing
    if (!valid(a, ids[i]) || a->refs[(size_t)ids[i]] == 0)
      return record_error(PKV_EINVAL, "%s: block %d is not allocated", fn, ids[i]);
  for (int32_t i = 0; i < n; ++i) ++a->refs[(size_t)ids[i]];
  return PKV_OK;
}

int pkv_allocator_release(pkv_block_allocator* a, const int32_t* ids, int32_t n) {
  const char* fn = "pkv_allocator_release";
  if (a == nullptr || (n > 0 && ids == nullptr) || n < 0)
    return record_error(PKV_EINVAL, "%s: null allocator/ids or n = %d", fn, n);
  std::lock_guard<std::mutex> lock(a->mu);
  // all or nothing, counting repeats of one id within the list
  std::vector<int32_t> need;
  for (int32_t i = 0; i < n; ++i) {
    if (!valid(a, ids[i]))
      return record_error(PKV_EINVAL, "%s: block %d out of range", fn, ids[i]);
    int32_t seen = 1;
    for (int32_t k = 0; k < i; ++k) seen += ids[k] == ids[i];
    if (seen > a->refs[(size_t)ids[i]])
      return record_error(PKV_EINVAL, "%s: block %d released more often than held", fn, ids[i]);
  }
  for (int32_t i = 0; i < n; ++i)
    if (--a->refs[(size_t)ids[i]] == 0) a->free.push_back(ids[i]);
  return PKV_OK;
}

int pkv_allocator_prepare_write(pkv_block_allocator* a, int32_t* table_row, int32_t first,
                                int32_t last, int32_t* src_ids, int32_t* dst_ids,
                                int32_t* num_copies) {
  const char* fn = "pkv_allocator_prepare_write";
  if (a == nullptr || table_row == nullptr || num_copies == nullptr || first < 0 || last < first)
    return record_error(PKV_EINVAL, "%s: null argument or range [%d, %d]", fn, first, last);
  *num_copies = 0;
  std::lock_guard<std::mutex> lock(a->mu);
  int32_t shared = 0;
  for (int32_t j = first; j <= last; ++j) {
    const int32_t id = table_row[j];
    if (!valid(a, id) || a->refs[(size_t)id] == 0)
      return record_error(PKV_EINVAL, "%s: table entry %d holds unallocated block %d", fn, j, id);
    for (int32_t k = first; k < j; ++k)
      if (table_row[k] == id)
        return record_error(PKV_EINVAL, "%s: block %d appears twice in the range", fn, id);
    shared += a->refs[(size_t)id] > 1;
  }
  if (shared > 0 && (src_ids == nullptr || dst_ids == nullptr))
    return record_error(PKV_EINVAL, "%s: %d copies needed, no arrays to report them", fn, shared);
  if ((size_t)shared > a->free.size())
    return record_error(PKV_ENOMEM, "%s: %d private copies needed, %zu blocks free", fn, shared,
                        a->free.size());
  int32_t n = 0;
  for (int32_t j = first; j <= last; ++j) {
    const int32_t id = table_row[j];
    if (a->refs[(size_t)id] <= 1) continue;
    const int32_t fresh = a->free.back();
    a->free.pop_back();
    a->refs[(size_t)fresh] = 1;
    --a->refs[(size_t)id];  // stays >= 1: the other holders keep it
    src_ids[n] = id;
    dst_ids[n] = fresh;
    table_row[j] = fresh;
    ++n;
  }
  *num_copies = n;
  return PKV_OK;
}

}  // extern "C"
