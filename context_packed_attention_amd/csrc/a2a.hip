// The hierarchical (a2a + p2p) front end's all-to-all for one a2a group,
// played on one device ("Hybrid / Hierarchical Context Parallel Skill",
// sections "Enablement" and "Implementation Map": CP = a2a size x p2p size,
// every padded length divisible by 2*CP). The a2a groups are runs of
// consecutive CP ranks, CP rank c = p * A + a; the group's chunks are then
// the p2p-level chunk pair (p, 2P-1-p), a p2p-level chunk being A
// consecutive CP-level chunks. Forward: A sequence-split, all-head local
// tensors -> A head-split tensors in p2p rank p's local layout. Inverse: the
// way back (for gradients). Pure data movement, HBM-bound: one wavefront per
// output row, 16 bytes per lane.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "cp_attn.h"
#include "internal.h"
#include "kern_common.h"

namespace cpattn {

struct A2APtrs {
  const uint4* in[CP_ATTN_MAX_CP];
  uint4* out[CP_ATTN_MAX_CP];
};

// sequence holding CP-local row t: the last b with cupl[b] <= t < cupl[b+1]
__device__ __forceinline__ int seq_of(const int32_t* cupl, int B, int t) {
  int lo = 0, hi = B;  // cupl[lo] <= t < cupl[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cupl[mid] <= t)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// p2p-local row tp (in units of CP-local rows scaled by A) -> (source CP
// rank a within the group, CP-local row)
__device__ __forceinline__ void p2p_row_source(const int32_t* cupl, int B, int A, int tp, int& a, int& t_cp) {
  // p2p-local sequence starts are A * cupl[b]
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (A * cupl[mid] <= tp)
      lo = mid;
    else
      hi = mid;
  }
  const int base = cupl[lo];
  const int c = (cupl[lo + 1] - base) >> 1;  // CP chunk rows of this sequence
  const int o = tp - A * base;
  if (o < A * c) {  // CP chunk pA + j: first chunk of CP rank pA + j
    const int j = o / c;
    a = j;
    t_cp = base + (o - j * c);
  } else {  // mirrored chunk: second chunk of CP rank pA + A-1-j
    const int o2 = o - A * c;
    const int j = o2 / c;
    a = A - 1 - j;
    t_cp = base + c + (o2 - j * c);
  }
}

// out[a'][tp] = heads [a' H/A, (a'+1) H/A) of in[a][t_cp], tp over the A * T_local p2p-local rows
__global__ void __launch_bounds__(256) a2a_seq_to_head_kernel(A2APtrs ptr, const int32_t* __restrict__ cupl, int B,
                                                              int A, int t_local, int units_in_row, int units_out) {
  const int lane = threadIdx.x & 63;
  const long long rows = (long long)A * A * t_local;  // (a', tp) pairs
  const long long wave = (blockIdx.x * (long long)blockDim.x + threadIdx.x) >> 6;
  const long long nwaves = ((long long)gridDim.x * blockDim.x) >> 6;
  for (long long r = wave; r < rows; r += nwaves) {
    const int ao = (int)(r / ((long long)A * t_local));
    const int tp = (int)(r - (long long)ao * A * t_local);
    int a, t_cp;
    p2p_row_source(cupl, B, A, tp, a, t_cp);
    const uint4* src = ptr.in[a] + (long long)t_cp * units_in_row + (long long)ao * units_out;
    wave_copy(src, ptr.out[ao] + (long long)tp * units_out, units_out, lane);
  }
}

// the inverse: out[a][t_cp] (all heads) from in[a'][tp] for every a'
__global__ void __launch_bounds__(256) a2a_head_to_seq_kernel(A2APtrs ptr, const int32_t* __restrict__ cupl, int B,
                                                              int A, int t_local, int units_in, int units_out_row) {
  const int lane = threadIdx.x & 63;
  const long long rows = (long long)A * t_local;  // (a, t_cp) pairs
  const long long wave = (blockIdx.x * (long long)blockDim.x + threadIdx.x) >> 6;
  const long long nwaves = ((long long)gridDim.x * blockDim.x) >> 6;
  for (long long r = wave; r < rows; r += nwaves) {
    const int a = (int)(r / t_local);
    const int t_cp = (int)(r - (long long)a * t_local);
    const int b = seq_of(cupl, B, t_cp);
    const int base = cupl[b];
    const int c = (cupl[b + 1] - base) >> 1;
    const int o = t_cp - base;
    const int tp = o < c ? A * base + a * c + o : A * base + (2 * A - 1 - a) * c + (o - c);
    uint4* dst = ptr.out[a] + (long long)t_cp * units_out_row;
    for (int ao = 0; ao < A; ++ao)
      wave_copy(ptr.in[ao] + (long long)tp * units_in, dst + (long long)ao * units_in, units_in, lane);
  }
}

static unsigned a2a_grid(long long rows) {
  const long long waves_per_block = 4;
  long long b = (rows + waves_per_block - 1) / waves_per_block;
  return (unsigned)std::max<long long>(1, std::min<long long>(b, 8192));
}

static cp_attn_status a2a_check(const cp_attn_meta* m, int32_t a2a_size, int32_t p2p_rank, int32_t heads,
                                int32_t head_bytes, const void* const* in, void* const* out) {
  if (!m) return fail(CP_ATTN_ERR_INVALID_ARG, "meta is NULL");
  if (a2a_size < 1 || m->cp % a2a_size != 0)
    return fail(CP_ATTN_ERR_INVALID_ARG, "a2a_size must divide the metadata's cp_size");
  if (p2p_rank < 0 || p2p_rank >= m->cp / a2a_size) return fail(CP_ATTN_ERR_INVALID_ARG, "p2p_rank out of range");
  if (heads <= 0 || heads % a2a_size != 0) return fail(CP_ATTN_ERR_INVALID_ARG, "heads must be a positive multiple of a2a_size");
  if (head_bytes <= 0 || head_bytes % 16 != 0) return fail(CP_ATTN_ERR_INVALID_ARG, "head_bytes must be a positive multiple of 16");
  if (!in || !out) return fail(CP_ATTN_ERR_INVALID_ARG, "NULL pointer array");
  for (int a = 0; a < a2a_size; ++a) {
    if (!in[a] || !out[a]) return fail(CP_ATTN_ERR_INVALID_ARG, "NULL tensor pointer");
    if ((((uintptr_t)in[a]) | ((uintptr_t)out[a])) & 15) return fail(CP_ATTN_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  }
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != m->device)
    return fail(CP_ATTN_ERR_INVALID_ARG, "current device differs from the metadata's device");
  return CP_ATTN_OK;
}

}  // namespace cpattn

using namespace cpattn;

extern "C" cp_attn_status cp_attn_a2a_seq_to_head(const cp_attn_meta* m, int32_t a2a_size, int32_t p2p_rank,
                                                  int32_t heads, int32_t head_bytes, const void* const* in,
                                                  void* const* out, void* stream) {
  set_error("");
  cp_attn_status rc = a2a_check(m, a2a_size, p2p_rank, heads, head_bytes, in, out);
  if (rc != CP_ATTN_OK) return rc;
  const int tl = m->sum.t_local;
  if (tl == 0) return CP_ATTN_OK;
  A2APtrs ptr{};
  for (int a = 0; a < a2a_size; ++a) {
    ptr.in[a] = (const uint4*)in[a];
    ptr.out[a] = (uint4*)out[a];
  }
  const int units_in_row = heads * (head_bytes / 16);
  const int units_out = units_in_row / a2a_size;
  hipStream_t st = (hipStream_t)stream;
  timing_begin(st, "a2a_seq_to_head");
  hipLaunchKernelGGL(a2a_seq_to_head_kernel, dim3(a2a_grid((long long)a2a_size * a2a_size * tl)), dim3(256), 0, st, ptr,
                     (const int32_t*)(m->d_tab + m->lay.cupl), m->B, a2a_size, tl, units_in_row, units_out);
  timing_end(st);
  return hip_check(hipGetLastError(), "a2a_seq_to_head launch");
}

extern "C" cp_attn_status cp_attn_a2a_head_to_seq(const cp_attn_meta* m, int32_t a2a_size, int32_t p2p_rank,
                                                  int32_t heads, int32_t head_bytes, const void* const* in,
                                                  void* const* out, void* stream) {
  set_error("");
  cp_attn_status rc = a2a_check(m, a2a_size, p2p_rank, heads, head_bytes, in, out);
  if (rc != CP_ATTN_OK) return rc;
  const int tl = m->sum.t_local;
  if (tl == 0) return CP_ATTN_OK;
  A2APtrs ptr{};
  for (int a = 0; a < a2a_size; ++a) {
    ptr.in[a] = (const uint4*)in[a];
    ptr.out[a] = (uint4*)out[a];
  }
  const int units_out_row = heads * (head_bytes / 16);
  const int units_in = units_out_row / a2a_size;
  hipStream_t st = (hipStream_t)stream;
  timing_begin(st, "a2a_head_to_seq");
  hipLaunchKernelGGL(a2a_head_to_seq_kernel, dim3(a2a_grid((long long)a2a_size * tl)), dim3(256), 0, st, ptr,
                     (const int32_t*)(m->d_tab + m->lay.cupl), m->B, a2a_size, tl, units_in, units_out_row);
  timing_end(st);
  return hip_check(hipGetLastError(), "a2a_head_to_seq launch");
}
