// One rank share captured into a HIP graph: the metadata is built once per
// batch, then the forward and backward launches of the share replay with one
// graph launch ("[PyTorch][Attention] THD P2P context-parallel regression
// ...", sections "Describe the bug" and "Expected behavior": launch gaps on
// the main stream, graph-safe padding metadata).
#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "cp_attn.h"
#include "internal.h"

struct cp_attn_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int device = -1;
  int64_t kernels = 0;
};

using namespace cpattn;

namespace {
void destroy(cp_attn_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}
}  // namespace

extern "C" cp_attn_status cp_attn_graph_capture(const cp_attn_meta* m, int32_t passes, const void* q,
                                                const void* const* k_shards, const void* const* v_shards,
                                                int32_t hq, int32_t hkv, int32_t d, float softmax_scale,
                                                int32_t causal, void* out, float* lse, const void* dout, void* dq,
                                                void* const* dk_parts, void* const* dv_parts, void* ws_fwd,
                                                size_t ws_fwd_bytes, void* ws_bwd, size_t ws_bwd_bytes,
                                                cp_attn_graph** out_graph) {
  set_error("");
  if (!out_graph) return fail(CP_ATTN_ERR_INVALID_ARG, "out_graph is NULL");
  *out_graph = nullptr;
  if (!m) return fail(CP_ATTN_ERR_INVALID_ARG, "meta is NULL");
  if (passes < 1 || passes > 3) return fail(CP_ATTN_ERR_INVALID_ARG, "passes must be 1, 2 or 3");
  int dev = -1;
  cp_attn_status rc = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc != CP_ATTN_OK) return rc;
  hipStream_t cs = nullptr;
  if ((rc = hip_check(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking), "hipStreamCreate(capture)")) != CP_ATTN_OK)
    return rc;
  cp_attn_graph* g = new cp_attn_graph();
  g->device = dev;
  rc = hip_check(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture");
  if (rc == CP_ATTN_OK) {
    cp_attn_status crc = CP_ATTN_OK;
    if (passes & 1)
      crc = cp_attn_fwd(m, q, k_shards, v_shards, hq, hkv, d, softmax_scale, causal, out, lse, ws_fwd, ws_fwd_bytes,
                        cs);
    if (crc == CP_ATTN_OK && (passes & 2))
      crc = cp_attn_bwd(m, q, k_shards, v_shards, out, lse, dout, hq, hkv, d, softmax_scale, causal, dq, dk_parts,
                        dv_parts, ws_bwd, ws_bwd_bytes, cs);
    // end the capture in every case, keeping the first error's message
    const char* msg = cp_attn_last_error();
    std::string keep = msg ? msg : "";
    const hipError_t e = hipStreamEndCapture(cs, &g->graph);
    if (crc != CP_ATTN_OK) {
      rc = fail(crc, keep.c_str());
    } else {
      rc = hip_check(e, "hipStreamEndCapture");
    }
  }
  if (rc == CP_ATTN_OK) rc = hip_check(hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0), "hipGraphInstantiate");
  if (rc == CP_ATTN_OK) {
    size_t n = 0;
    rc = hip_check(hipGraphGetNodes(g->graph, nullptr, &n), "hipGraphGetNodes");
    if (rc == CP_ATTN_OK && n > 0) {
      std::vector<hipGraphNode_t> nodes(n);
      rc = hip_check(hipGraphGetNodes(g->graph, nodes.data(), &n), "hipGraphGetNodes");
      for (size_t i = 0; rc == CP_ATTN_OK && i < n; ++i) {
        hipGraphNodeType t;
        rc = hip_check(hipGraphNodeGetType(nodes[i], &t), "hipGraphNodeGetType");
        if (rc == CP_ATTN_OK && t == hipGraphNodeTypeKernel) ++g->kernels;
      }
    }
  }
  (void)hipStreamDestroy(cs);
  if (rc != CP_ATTN_OK) {
    destroy(g);
    return rc;
  }
  *out_graph = g;
  return CP_ATTN_OK;
}

extern "C" cp_attn_status cp_attn_graph_launch(const cp_attn_graph* g, void* stream) {
  set_error("");
  if (!g || !g->exec) return fail(CP_ATTN_ERR_INVALID_ARG, "graph is NULL");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != g->device)
    return fail(CP_ATTN_ERR_INVALID_ARG, "current device differs from the graph's device");
  return hip_check(hipGraphLaunch(g->exec, (hipStream_t)stream), "hipGraphLaunch");
}

extern "C" int64_t cp_attn_graph_kernels(const cp_attn_graph* g) { return g ? g->kernels : 0; }

extern "C" void cp_attn_graph_free(cp_attn_graph* g) {
  if (!g) return;
  const int dev = g->device;
  int cur = -1;
  const bool switched = hipGetDevice(&cur) == hipSuccess && cur != dev && hipSetDevice(dev) == hipSuccess;
  (void)hipDeviceSynchronize();
  destroy(g);
  if (switched) (void)hipSetDevice(cur);
}
