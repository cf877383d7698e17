// Internal declarations shared by the HIP translation units of libcpattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/cp_attn.h"

namespace cpattn {

// ---------------------------------------------------------------- tiling
// Wavefronts per block of the attention kernels; each owns 32 query rows
// (forward, dQ) or 32 key rows (dK/dV).
#ifndef CPA_NWAVES
#define CPA_NWAVES 4
#endif
constexpr int NWAVES = CPA_NWAVES;
constexpr int BLOCK_THREADS = 64 * NWAVES;
// Query rows per forward / dQ work item.
constexpr int FWD_BM = 32 * NWAVES;
// Key rows per dK/dV work item.
#ifndef CPA_DKDV_KB
#define CPA_DKDV_KB 1
#endif
// 32-key blocks per dK/dV wavefront; the dK/dV block covers DKDV_BN keys
constexpr int DKDV_KB = CPA_DKDV_KB;
constexpr int DKDV_BN = 32 * NWAVES * DKDV_KB;
// Work lists up to this length are sorted heaviest-first on the device.
constexpr int SORT_CAP = 4096;

// Device summary words (int32), written by the metadata kernel.
enum SummaryWord : int {
  SW_ERR = 0,
  SW_PAD = 1,
  SW_TLOCAL = 2,
  SW_HAS_TAIL = 3,
  SW_VALID_ROWS = 4,
  SW_TILES_FWD = 8,                       // + step
  SW_TILES_DKDV = SW_TILES_FWD + CP_ATTN_MAX_CP,
  SW_KIND = SW_TILES_DKDV + CP_ATTN_MAX_CP,
  SW_SRC = SW_KIND + CP_ATTN_MAX_CP,
  SW_COUNT = SW_SRC + CP_ATTN_MAX_CP
};

// Error bits in SW_ERR.
enum MetaErr : int {
  ME_START = 1,        // cu[0] or cup[0] != 0
  ME_CU_ORDER = 2,     // cu decreasing
  ME_CUP_ORDER = 4,    // cup decreasing
  ME_LEN = 8,          // L_b > P_b
  ME_DIV = 16,         // P_b % (2 CP) != 0
  ME_ALLOC = 32,       // t_alloc < T_local
  ME_HINT = 64,        // pad hint contradicts the values
  ME_RANGE = 128       // T_local does not fit 31-bit row indices
};

// Row flags of the rank's local rows (rowflags table).
enum RowFlag : int { RF_VALID = 1, RF_SECOND = 2 };

// Offsets (in int32 elements) of the device tables inside one allocation.
struct MetaLayout {
  int64_t cu, cup, chunk, cupl, cuph;
  int64_t cu_full, cu_first, cu_second;  // + s * (B + 1)
  int64_t steps;                         // + i * 4 * B: q_start, q_len, kv_start, kv_len
  int64_t rowflags;                      // [t_alloc]
  int64_t fwd_off, dkdv_off;             // per-step per-sequence tile offsets: + i * (B + 1)
  int64_t fwd_tiles, dkdv_tiles;         // + i * cap * 2 : (b, tile) pairs
  int64_t fwd_keys, dkdv_keys;           // + i * cap : sort keys (scratch)
  int64_t summary;                       // [SW_COUNT]
  int64_t fwd_cap, dkdv_cap;
  int64_t total;
};

MetaLayout make_layout(int B, int cp, int64_t t_alloc);

}  // namespace cpattn

struct cp_attn_meta {
  int device;
  int B, cp, rank, pad_hint;
  int64_t t_alloc;
  cpattn::MetaLayout lay;
  int32_t* d_tab;    // device tables
  size_t tab_bytes;  // size of the d_tab buffer (from the per-device pool)
  cp_attn_summary sum;
};

namespace cpattn {

// side streams of the calling thread (streams.hip)
constexpr int MAX_SIDE = 1;
struct SideSet {
  bool ready = false;
  hipStream_t s[MAX_SIDE] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[MAX_SIDE] = {};
};
cp_attn_status side_set(int device, SideSet** out);
cp_attn_status fork_to(SideSet* ss, hipStream_t st, int n);
cp_attn_status join_from(SideSet* ss, hipStream_t st, int n);
int cu_count(int device);
// launches this short (under four full waves of two blocks per compute
// unit) leave tails that concurrent independent launches can fill
bool short_launches(long long max_blocks, int device);

// whether the backward runs its dK/dV and dQ launches concurrently (bwd.hip)
bool bwd_forks(const cp_attn_meta* m, int hq);

// per-kernel event timing (no-ops unless enabled through the C ABI)
void timing_begin(hipStream_t st, const char* name);
void timing_end(hipStream_t st);

// thread-local error message
void set_error(const std::string& msg);
cp_attn_status fail(cp_attn_status st, const std::string& msg);
cp_attn_status hip_check(hipError_t e, const char* what);

inline const int32_t* tab(const cp_attn_meta* m, int64_t off) { return m->d_tab + off; }

// Step table accessors (device pointers)
struct StepTab {
  const int32_t* q_start;
  const int32_t* q_len;
  const int32_t* kv_start;
  const int32_t* kv_len;
};
inline StepTab step_tab(const cp_attn_meta* m, int i) {
  const int32_t* base = m->d_tab + m->lay.steps + (int64_t)i * 4 * m->B;
  return StepTab{base, base + m->B, base + 2 * m->B, base + 3 * m->B};
}

}  // namespace cpattn
