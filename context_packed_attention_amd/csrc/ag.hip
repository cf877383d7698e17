// All-gather context parallelism on one device: the rank holds its own query
// chunks and the whole gathered K/V ("Hybrid / Hierarchical Context Parallel
// Skill", Implementation Map: cp_comm_type "all_gather"), and produces its
// queries' outputs plus its contribution to the gradient of every gathered
// key row (what a reduce-scatter would then sum across ranks).
//
// The pairs a rank's queries attend to are the same whatever the exchange:
// its two chunks against every key of their sequence at or before them. The
// ring-step kernels already cover exactly those pairs, one source shard at a
// time, so the all-gather share is computed as: gather the CP shard views out
// of the gathered K/V (one HBM-bound permutation), run the ring steps, and
// scatter the per-shard dK/dV parts back to gathered rows. Every gathered row
// belongs to exactly one shard, so the scatter is a permutation too: no
// accumulation and no extra rounding.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "internal.h"
#include "kern_common.h"

namespace cpattn {
namespace {

// last index j in [0, n] with a[j] <= x (a non-decreasing, a[0] <= x)
__device__ __forceinline__ int last_le(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// gathered row of local row t of shard s (chunks s and 2 CP - 1 - s of each
// sequence, in order)
__device__ __forceinline__ long long gathered_row(const int32_t* tab, const MetaLayout& L, int B, int cp, int s, int t) {
  const int32_t* cupl = tab + L.cupl;
  int b = last_le(cupl, B, t);
  if (b >= B) b = B - 1;
  while (b > 0 && cupl[b] == cupl[b + 1]) --b;  // skip empty sequences
  const int o = t - cupl[b];
  const int c = tab[L.chunk + b];
  const int k = o < c ? s : 2 * cp - 1 - s;
  return (long long)tab[L.cup + b] + (long long)k * c + (o < c ? o : o - c);
}

// One wavefront per (shard, local row): the row's gathered position is found
// once, then K and V (or dK and dV) rows are copied 16 bytes per lane.
// shards[s][t] = full[gathered_row(s, t)] (gather) or the reverse (scatter).
template <bool GATHER>
__global__ void __launch_bounds__(256) ag_permute_kernel(const int32_t* __restrict__ tab, MetaLayout L, int B, int cp,
                                                         const uint4* __restrict__ a_src, const uint4* __restrict__ b_src,
                                                         uint4* __restrict__ a_dst, uint4* __restrict__ b_dst,
                                                         long long shard_units, int upr, int t_local) {
  const int lane = threadIdx.x & 63;
  const long long rows = (long long)cp * t_local;
  const long long wave = (blockIdx.x * (long long)blockDim.x + threadIdx.x) >> 6;
  const long long nwaves = ((long long)gridDim.x * blockDim.x) >> 6;
  for (long long r = wave; r < rows; r += nwaves) {
    const int s = (int)(r / t_local);
    const int t = (int)(r - (long long)s * t_local);
    const long long g = gathered_row(tab, L, B, cp, s, t) * upr;
    const long long l = s * shard_units + (long long)t * upr;
    if (GATHER) {
      wave_copy(a_src + g, a_dst + l, upr, lane);
      wave_copy(b_src + g, b_dst + l, upr, lane);
    } else {
      wave_copy(a_src + l, a_dst + g, upr, lane);
      wave_copy(b_src + l, b_dst + g, upr, lane);
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// bytes of one shard-layout tensor of t_alloc rows
size_t shard_bytes(const cp_attn_meta* m, int hkv, int d) {
  return align256((size_t)std::max<int64_t>(m->t_alloc, 1) * hkv * d * 2);
}

// four wavefronts per block, one (shard, row) each
unsigned grid_for(long long rows) { return (unsigned)std::min<long long>(std::max<long long>((rows + 3) / 4, 1), 16384); }

cp_attn_status ag_check(const cp_attn_meta* m, const void* q, const void* k_full, const void* v_full, int hq, int hkv,
                        int d, const void* workspace) {
  if (!m) return fail(CP_ATTN_ERR_INVALID_ARG, "meta is NULL");
  if (!q || !k_full || !v_full) return fail(CP_ATTN_ERR_INVALID_ARG, "NULL tensor argument");
  if (hq <= 0 || hkv <= 0 || d <= 0) return fail(CP_ATTN_ERR_INVALID_ARG, "head counts and head_dim must be positive");
  if (((uintptr_t)k_full | (uintptr_t)v_full) & 15)
    return fail(CP_ATTN_ERR_INVALID_ARG, "gathered K/V must be 16-byte aligned");
  if (((long long)hkv * d * 2) % 16 != 0) return fail(CP_ATTN_ERR_UNSUPPORTED, "a K/V row must be a multiple of 16 bytes");
  if (workspace && ((uintptr_t)workspace & 255)) return fail(CP_ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return CP_ATTN_OK;
}

cp_attn_status ag_gather(const cp_attn_meta* m, const void* k_full, const void* v_full, char* k_sh, char* v_sh,
                         size_t sh_bytes, int hkv, int d, hipStream_t st) {
  const int tl = m->sum.t_local;
  const int upr = hkv * d * 2 / 16;
  timing_begin(st, "ag_gather");
  hipLaunchKernelGGL(ag_permute_kernel<true>, dim3(grid_for((long long)tl * m->cp)), dim3(256), 0, st, m->d_tab,
                     m->lay, m->B, m->cp, (const uint4*)k_full, (const uint4*)v_full, (uint4*)k_sh, (uint4*)v_sh,
                     (long long)(sh_bytes / 16), upr, tl);
  timing_end(st);
  return hip_check(hipGetLastError(), "ag_gather launch");
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" {

size_t cp_attn_ag_workspace_bytes(const cp_attn_meta* m, int32_t hq, int32_t hkv, int32_t d, int32_t pass) {
  if (!m || hq <= 0 || hkv <= 0 || d <= 0 || (pass != 0 && pass != 1)) return 0;
  const size_t sh = shard_bytes(m, hkv, d) * m->cp;
  const size_t inner = align256(cp_attn_workspace_bytes(m, hq, hkv, d, pass));
  return (pass == 0 ? 2 : 4) * sh + inner;  // K, V shards (+ dK, dV parts) + the ring steps' workspace
}

cp_attn_status cp_attn_ag_fwd(const cp_attn_meta* m, const void* q, const void* k_full, const void* v_full,
                              int32_t hq, int32_t hkv, int32_t d, float softmax_scale, int32_t causal, void* out,
                              float* lse, void* workspace, size_t ws_bytes, void* stream) {
  set_error("");
  cp_attn_status rc = ag_check(m, q, k_full, v_full, hq, hkv, d, workspace);
  if (rc != CP_ATTN_OK) return rc;
  const size_t need = cp_attn_ag_workspace_bytes(m, hq, hkv, d, 0);
  if (!workspace || ws_bytes < need) return fail(CP_ATTN_ERR_WORKSPACE, "all-gather forward workspace missing or too small");
  if (m->cp > CP_ATTN_MAX_CP) return fail(CP_ATTN_ERR_UNSUPPORTED, "cp_size too large");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != m->device)
    return fail(CP_ATTN_ERR_INVALID_ARG, "current device differs from the metadata's device");
  hipStream_t st = (hipStream_t)stream;
  const size_t sb = shard_bytes(m, hkv, d);
  char* ws = (char*)workspace;
  char* k_sh = ws;
  char* v_sh = ws + sb * m->cp;
  char* inner = ws + 2 * sb * m->cp;
  const void* ks[CP_ATTN_MAX_CP];
  const void* vs[CP_ATTN_MAX_CP];
  for (int s = 0; s < m->cp; ++s) {
    ks[s] = k_sh + s * sb;
    vs[s] = v_sh + s * sb;
  }
  if (m->sum.t_local > 0 && (rc = ag_gather(m, k_full, v_full, k_sh, v_sh, sb, hkv, d, st)) != CP_ATTN_OK) return rc;
  return cp_attn_fwd(m, q, ks, vs, hq, hkv, d, softmax_scale, causal, out, lse, inner, ws_bytes - (inner - ws), stream);
}

cp_attn_status cp_attn_ag_bwd(const cp_attn_meta* m, const void* q, const void* k_full, const void* v_full,
                              const void* out, const float* lse, const void* dout, int32_t hq, int32_t hkv, int32_t d,
                              float softmax_scale, int32_t causal, void* dq, void* dk_full, void* dv_full,
                              void* workspace, size_t ws_bytes, void* stream) {
  set_error("");
  cp_attn_status rc = ag_check(m, q, k_full, v_full, hq, hkv, d, workspace);
  if (rc != CP_ATTN_OK) return rc;
  if (!dk_full || !dv_full) return fail(CP_ATTN_ERR_INVALID_ARG, "NULL gradient output");
  if (((uintptr_t)dk_full | (uintptr_t)dv_full) & 15)
    return fail(CP_ATTN_ERR_INVALID_ARG, "gathered dK/dV must be 16-byte aligned");
  const size_t need = cp_attn_ag_workspace_bytes(m, hq, hkv, d, 1);
  if (!workspace || ws_bytes < need) return fail(CP_ATTN_ERR_WORKSPACE, "all-gather backward workspace missing or too small");
  if (m->cp > CP_ATTN_MAX_CP) return fail(CP_ATTN_ERR_UNSUPPORTED, "cp_size too large");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != m->device)
    return fail(CP_ATTN_ERR_INVALID_ARG, "current device differs from the metadata's device");
  hipStream_t st = (hipStream_t)stream;
  const size_t sb = shard_bytes(m, hkv, d);
  char* ws = (char*)workspace;
  char* k_sh = ws;
  char* v_sh = ws + sb * m->cp;
  char* dk_sh = ws + 2 * sb * m->cp;
  char* dv_sh = ws + 3 * sb * m->cp;
  char* inner = ws + 4 * sb * m->cp;
  const void* ks[CP_ATTN_MAX_CP];
  const void* vs[CP_ATTN_MAX_CP];
  void* dks[CP_ATTN_MAX_CP];
  void* dvs[CP_ATTN_MAX_CP];
  for (int s = 0; s < m->cp; ++s) {
    ks[s] = k_sh + s * sb;
    vs[s] = v_sh + s * sb;
    dks[s] = dk_sh + s * sb;
    dvs[s] = dv_sh + s * sb;
  }
  const int tl = m->sum.t_local;
  if (tl > 0 && (rc = ag_gather(m, k_full, v_full, k_sh, v_sh, sb, hkv, d, st)) != CP_ATTN_OK) return rc;
  rc = cp_attn_bwd(m, q, ks, vs, out, lse, dout, hq, hkv, d, softmax_scale, causal, dq, dks, dvs, inner,
                   ws_bytes - (inner - ws), stream);
  if (rc != CP_ATTN_OK || tl == 0) return rc;
  const int upr = hkv * d * 2 / 16;
  timing_begin(st, "ag_scatter");
  hipLaunchKernelGGL(ag_permute_kernel<false>, dim3(grid_for((long long)tl * m->cp)), dim3(256), 0, st, m->d_tab,
                     m->lay, m->B, m->cp, (const uint4*)dk_sh, (const uint4*)dv_sh, (uint4*)dk_full, (uint4*)dv_full,
                     (long long)(sb / 16), upr, tl);
  timing_end(st);
  return hip_check(hipGetLastError(), "ag_scatter launch");
}

}  // extern "C"
