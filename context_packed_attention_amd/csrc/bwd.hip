// Backward of one CP rank's share (filled in below).
#include <hip/hip_runtime.h>

#include "internal.h"

using namespace cpattn;

extern "C" cp_attn_status cp_attn_bwd(const cp_attn_meta* m, const void* q, const void* const* k_shards,
                                      const void* const* v_shards, const void* out, const float* lse,
                                      const void* dout, int32_t hq, int32_t hkv, int32_t d, float softmax_scale,
                                      int32_t causal, void* dq, void* const* dk_parts, void* const* dv_parts,
                                      void* workspace, size_t ws_bytes, void* stream) {
  return fail(CP_ATTN_ERR_UNSUPPORTED, "backward not built yet");
}
