// A decode tick captured once into a HIP graph, for one batch-size bucket.
//
// Pages: "Inference Server" (project README mirror), section "The engine" --
// the engine replays decode steps captured per batch-size bucket, since a
// small decode call costs little more than its launch; "Inference Server --
// Architecture Map", section "How a single request flows through the
// system" -- one batched decode per tick.
//
// The graph holds one paged_attn_decode_append launch over fixed buffers
// (q, the new rows, tables, lengths, outputs) sized for the bucket; lengths
// and tables are read by the kernel when it runs, so one capture serves every
// tick whose sequences fit the bucket (unused rows carry length 0 and are
// skipped).  The decode workspace belongs to the graph: allocated and
// zero-filled at creation, outside the capture, so the graph holds no
// memset node.
#include <hip/hip_runtime.h>

#include <new>

#include "launch.hpp"
#include "pkv.h"

using pkv::record_error;

struct pkv_decode_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  void* workspace = nullptr;
};

extern "C" {

void pkv_decode_graph_destroy(pkv_decode_graph* g) {
  if (g == nullptr) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  if (g->workspace) (void)hipFree(g->workspace);
  delete g;
}

int pkv_decode_graph_create(pkv_decode_graph** graph, void* out, float* lse, const void* q,
                            const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                            int32_t num_blocks, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, int32_t num_seqs, int32_t num_kv_heads,
                            int32_t gqa_group, int32_t head_dim, int32_t block_size, float scale,
                            float softcap, int32_t window, int32_t partition_size, int32_t dtype) {
  const char* fn = "pkv_decode_graph_create";
  if (graph == nullptr) return record_error(PKV_EINVAL, "%s: graph is null", fn);
  *graph = nullptr;
  if (num_seqs < 1) return record_error(PKV_EINVAL, "%s: a bucket needs num_seqs >= 1", fn);
  const size_t ws_bytes = paged_attn_decode_workspace_size(
      num_seqs, num_kv_heads, gqa_group, head_dim, max_context_len, partition_size);
  if (ws_bytes == 0)
    return record_error(PKV_EINVAL, "%s: invalid sizes (num_seqs %d, kv heads %d, group %d, "
                      "head_dim %d, max_context_len %d, partition_size %d)", fn, num_seqs,
                      num_kv_heads, gqa_group, head_dim, max_context_len, partition_size);
  pkv_decode_graph* g = new (std::nothrow) pkv_decode_graph();
  if (g == nullptr) return record_error(PKV_ENOMEM, "%s: out of host memory", fn);

  hipStream_t s = nullptr;
  hipError_t e = hipMalloc(&g->workspace, ws_bytes);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipMemsetAsync(g->workspace, 0, ws_bytes, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    if (s) (void)hipStreamDestroy(s);
    pkv_decode_graph_destroy(g);
    return record_error(PKV_EHIP, "%s: %s", fn, hipGetErrorString(e));
  }

  e = hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(s);
    pkv_decode_graph_destroy(g);
    return record_error(PKV_EHIP, "%s: begin capture: %s", fn, hipGetErrorString(e));
  }
  const int rc = paged_attn_decode_append(
      out, lse, q, k_new, v_new, k_pool, v_pool, num_blocks, block_tables, max_blocks_per_seq,
      context_lens, max_context_len, num_seqs, num_kv_heads, gqa_group, head_dim, block_size,
      scale, softcap, window, partition_size, g->workspace, ws_bytes, dtype, s);
  const hipError_t ec = hipStreamEndCapture(s, &g->graph);  // always end the capture
  (void)hipStreamDestroy(s);
  if (rc != PKV_OK) {  // the call's own message stays in pkv_last_error
    pkv_decode_graph_destroy(g);
    return rc;
  }
  if (ec != hipSuccess) {
    pkv_decode_graph_destroy(g);
    return record_error(PKV_EHIP, "%s: end capture: %s", fn, hipGetErrorString(ec));
  }
  e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    pkv_decode_graph_destroy(g);
    return record_error(PKV_EHIP, "%s: instantiate: %s", fn, hipGetErrorString(e));
  }
  *graph = g;
  return PKV_OK;
}

int pkv_decode_graph_launch(pkv_decode_graph* g, struct ihipStream_t* stream) {
  if (g == nullptr || g->exec == nullptr)
    return record_error(PKV_EINVAL, "pkv_decode_graph_launch: graph is null");
  const hipError_t e = hipGraphLaunch(g->exec, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return record_error(PKV_EHIP, "pkv_decode_graph_launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // extern "C"
