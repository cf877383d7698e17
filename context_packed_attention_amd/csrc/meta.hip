// Per-rank packed-sequence metadata, built on the device.
//
// "[PyTorch][Attention] THD P2P context-parallel regression when padded
// cu_seqlens are value-equal but not object-identical", "Describe the bug":
// the per-rank sequence lengths of every ring step were recomputed by a
// helper that launched thousands of small kernels, and the padded path was
// chosen from object identity. Here one group of four small kernels builds
// every table once per batch, and the padding decision is a comparison of
// values ("Expected behavior"). "Hybrid / Hierarchical Context Parallel
// Skill", "Enablement": padded lengths divide by 2*CP.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace cpattn {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

cp_attn_status fail(cp_attn_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

cp_attn_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return CP_ATTN_OK;
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return CP_ATTN_ERR_HIP;
}

MetaLayout make_layout(int B, int cp, int64_t t_alloc) {
  MetaLayout L{};
  int64_t o = 0;
  auto take = [&](int64_t n) {
    int64_t at = o;
    o += (n + 63) & ~int64_t(63);  // 256-byte aligned sections
    return at;
  };
  L.cu = take(B + 1);
  L.cup = take(B + 1);
  L.chunk = take(B);
  L.cupl = take(B + 1);
  L.cuph = take(B + 1);
  L.cu_full = take((int64_t)cp * (B + 1));
  L.cu_first = take((int64_t)cp * (B + 1));
  L.cu_second = take((int64_t)cp * (B + 1));
  L.steps = take((int64_t)cp * 4 * B);
  L.rowflags = take(t_alloc > 0 ? t_alloc : 1);
  L.fwd_off = take((int64_t)cp * (B + 1));
  L.dkdv_off = take((int64_t)cp * (B + 1));
  L.fwd_cap = t_alloc / FWD_BM + B + 1;
  L.dkdv_cap = t_alloc / DKDV_BN + B + 1;
  L.fwd_tiles = take((int64_t)cp * L.fwd_cap * 2);
  L.dkdv_tiles = take((int64_t)cp * L.dkdv_cap * 2);
  L.fwd_keys = take((int64_t)cp * L.fwd_cap * 2);
  L.dkdv_keys = take((int64_t)cp * L.dkdv_cap * 2);
  L.summary = take(SW_COUNT);
  L.total = o;
  return L;
}

// ------------------------------------------------------------------ kernels

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// valid rows of chunk k when L valid tokens fill chunks of size c in order
__device__ __forceinline__ int chunk_valid(int L, int c, int k) { return clampi(L - k * c, 0, c); }

// Block-wide exclusive scan over 256 threads (four wavefronts: a shuffle scan
// within each, then the wavefront totals through LDS); returns the exclusive
// prefix and writes the block total to *total. Two barriers; `sm` holds at
// least 4 ints and may be reused right after the call.
__device__ int block_excl_scan256(int v, int* sm, int* total) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sm[wv] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int w = sm[k];
    before += k < wv ? w : 0;
    tot += w;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Where the tables kernel reads cu_seqlens / cu_seqlens_padded: device
// arrays (cup NULL = no padding), or the values themselves carried in the
// kernel's arguments (the host path, B <= CP_ATTN_HOST_META_MAX_B).
struct DevSeqlens {
  const int32_t* cu;
  const int32_t* cup;
  __device__ int a(int b) const { return cu[b]; }
  __device__ int p(int b) const { return cup ? cup[b] : cu[b]; }
};
struct ArgSeqlens {
  int32_t cu[CP_ATTN_HOST_META_MAX_B + 1];
  int32_t cup[CP_ATTN_HOST_META_MAX_B + 1];
  __device__ int a(int b) const { return cu[b]; }
  __device__ int p(int b) const { return cup[b]; }
};

// One block of 256 threads. Builds every per-sequence table, the validation
// word, the padding decision and the per-step work-item offsets.
template <class Src>
__global__ void __launch_bounds__(256) meta_tables_kernel(Src src, int B, int cp, int rank, int hint,
                                                          long long t_alloc, int32_t* __restrict__ tabp,
                                                          MetaLayout L) {
  __shared__ int sm[256];
  __shared__ int s_err, s_pad;
  __shared__ int s_carry[5 * CP_ATTN_MAX_CP];
  const int t = threadIdx.x;
  if (t == 0) {
    s_err = 0;
    s_pad = 0;
  }
  if (t < 5 * CP_ATTN_MAX_CP) s_carry[t] = 0;
  __syncthreads();
  int32_t* cu = tabp + L.cu;
  int32_t* cup = tabp + L.cup;
  // copy inputs + elementwise checks
  for (int b = t; b <= B; b += 256) {
    const int a = src.a(b), p = src.p(b);
    cu[b] = a;
    cup[b] = p;
    if (a != p) atomicOr(&s_pad, 1);
  }
  __syncthreads();
  if (t == 0 && (cu[0] != 0 || cup[0] != 0)) atomicOr(&s_err, ME_START);
  const int two_cp = 2 * cp;
  // kinds and sources of every step
  int kind_i[CP_ATTN_MAX_CP], src_i[CP_ATTN_MAX_CP];
  for (int i = 0; i < cp; ++i) {
    int s = ((rank - i) % cp + cp) % cp;
    src_i[i] = s;
    kind_i[i] = (i == 0) ? 0 : (s < rank ? 1 : 2);
  }
  int* cnt_carry = s_carry;  // [0, 3cp): lengths scans; [3cp, 4cp): fwd tiles; [4cp, 5cp): dkdv tiles
  for (int b0 = 0; b0 < B; b0 += 256) {
    const int b = b0 + t;
    const bool in = b < B;
    int Lb = 0, Pb = 0, c = 0, base = 0;
    if (in) {
      Lb = cu[b + 1] - cu[b];
      Pb = cup[b + 1] - cup[b];
      int e = 0;
      if (Lb < 0) e |= ME_CU_ORDER;
      if (Pb < 0) e |= ME_CUP_ORDER;
      if (Lb > Pb) e |= ME_LEN;
      if (Pb >= 0 && (Pb % two_cp) != 0) e |= ME_DIV;
      if (e) atomicOr(&s_err, e);
      if (Pb < 0) Pb = 0;
      Lb = clampi(Lb, 0, Pb);
      c = Pb / two_cp;
      base = cup[b] / cp;
      tabp[L.chunk + b] = c;
      tabp[L.cupl + b] = base;
      tabp[L.cuph + b] = cup[b] / two_cp;
    }
    // scans of the valid-row counts of every shard
    for (int s = 0; s < cp; ++s) {
      int f = in ? chunk_valid(Lb, c, s) : 0;
      int sc = in ? chunk_valid(Lb, c, two_cp - 1 - s) : 0;
      int vals[3] = {f + sc, f, sc};
      int64_t offs[3] = {L.cu_full, L.cu_first, L.cu_second};
      for (int k = 0; k < 3; ++k) {
        // every thread reads the carry before the scan's barriers, thread 0
        // updates it after them; the next read is in the next round of 256
        int tot;
        const int carry = cnt_carry[3 * s + k];
        const int ex = block_excl_scan256(vals[k], sm, &tot);
        if (in) tabp[offs[k] + (int64_t)s * (B + 1) + b] = carry + ex;
        if (t == 0) cnt_carry[3 * s + k] = carry + tot;
      }
    }
    // step tables and per-sequence work-item counts
    const int fr = chunk_valid(Lb, c, rank), sr = chunk_valid(Lb, c, two_cp - 1 - rank);
    for (int i = 0; i < cp; ++i) {
      const int kind = kind_i[i], s = src_i[i];
      const int fs = chunk_valid(Lb, c, s), ss = chunk_valid(Lb, c, two_cp - 1 - s);
      int q_start = base + (kind == 2 ? c : 0);
      int q_len = kind == 2 ? sr : fr + sr;
      int kv_len = kind == 1 ? fs : fs + ss;
      if (in) {
        int32_t* st = tabp + L.steps + (int64_t)i * 4 * B;
        st[b] = q_start;
        st[B + b] = q_len;
        st[2 * B + b] = base;
        st[3 * B + b] = kv_len;
      }
      int nf = in ? (q_len + FWD_BM - 1) / FWD_BM : 0;
      int nk = in ? (Pb / cp + DKDV_BN - 1) / DKDV_BN : 0;
      int tot;
      const int carry_f = cnt_carry[3 * cp + i];
      int ex = block_excl_scan256(nf, sm, &tot);
      if (in) tabp[L.fwd_off + (int64_t)i * (B + 1) + b] = carry_f + ex;
      if (t == 0) cnt_carry[3 * cp + i] = carry_f + tot;
      const int carry_k = cnt_carry[4 * cp + i];
      ex = block_excl_scan256(nk, sm, &tot);
      if (in) tabp[L.dkdv_off + (int64_t)i * (B + 1) + b] = carry_k + ex;
      if (t == 0) cnt_carry[4 * cp + i] = carry_k + tot;
    }
  }
  __syncthreads();
  if (t == 0) {
    int32_t* sw = tabp + L.summary;
    const int64_t tl = (int64_t)cup[B] / cp;
    int err = s_err;
    if (tl > t_alloc) err |= ME_ALLOC;
    if ((int64_t)cup[B] >= (1ll << 31) || tl >= (1ll << 30)) err |= ME_RANGE;
    if (hint >= 0 && hint != s_pad) err |= ME_HINT;
    tabp[L.cupl + B] = cup[B] / cp;
    tabp[L.cuph + B] = cup[B] / two_cp;
    for (int s = 0; s < cp; ++s) {
      tabp[L.cu_full + (int64_t)s * (B + 1) + B] = cnt_carry[3 * s];
      tabp[L.cu_first + (int64_t)s * (B + 1) + B] = cnt_carry[3 * s + 1];
      tabp[L.cu_second + (int64_t)s * (B + 1) + B] = cnt_carry[3 * s + 2];
    }
    sw[SW_ERR] = err;
    sw[SW_PAD] = s_pad;
    sw[SW_TLOCAL] = (int)tl;
    sw[SW_HAS_TAIL] = t_alloc > tl ? 1 : 0;
    sw[SW_VALID_ROWS] = cnt_carry[3 * rank];
    for (int i = 0; i < cp; ++i) {
      tabp[L.fwd_off + (int64_t)i * (B + 1) + B] = cnt_carry[3 * cp + i];
      tabp[L.dkdv_off + (int64_t)i * (B + 1) + B] = cnt_carry[4 * cp + i];
      sw[SW_TILES_FWD + i] = cnt_carry[3 * cp + i];
      sw[SW_TILES_DKDV + i] = cnt_carry[4 * cp + i];
      sw[SW_KIND + i] = kind_i[i];
      sw[SW_SRC + i] = src_i[i];
    }
  }
}

// last index j in [0, n] with a[j] <= x (a non-decreasing, a[0] <= x)
__device__ __forceinline__ int upper_idx(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;  // invariant a[lo] <= x
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Row flags of this rank's local rows: valid / in the second chunk.
__global__ void meta_rows_kernel(int32_t* __restrict__ tabp, MetaLayout L, int B, int cp, int rank,
                                 long long t_alloc) {
  const int32_t* sw = tabp + L.summary;
  if (sw[SW_ERR]) return;
  const int tl = sw[SW_TLOCAL];
  const int32_t* cupl = tabp + L.cupl;
  const int32_t* chunk = tabp + L.chunk;
  const int32_t* cf = tabp + L.cu_first + (int64_t)rank * (B + 1);
  const int32_t* cs = tabp + L.cu_second + (int64_t)rank * (B + 1);
  for (long long t = blockIdx.x * (long long)blockDim.x + threadIdx.x; t < t_alloc;
       t += (long long)gridDim.x * blockDim.x) {
    int f = 0;
    if (t < tl) {
      int b = upper_idx(cupl, B, (int)t);
      if (b >= B) b = B - 1;
      while (b > 0 && cupl[b] == cupl[b + 1]) --b;  // skip empty slots (never for t < tl)
      int o = (int)t - cupl[b];
      int c = chunk[b];
      if (o < c) {
        f = (o < cf[b + 1] - cf[b]) ? RF_VALID : 0;
      } else {
        f = RF_SECOND | ((o - c < cs[b + 1] - cs[b]) ? RF_VALID : 0);
      }
    }
    tabp[L.rowflags + t] = f;
  }
}

// Work items (sequence, tile) of every step, with a work estimate as sort key.
__global__ void meta_tiles_kernel(int32_t* __restrict__ tabp, MetaLayout L, int B, int cp) {
  const int32_t* sw = tabp + L.summary;
  if (sw[SW_ERR]) return;
  const int list = blockIdx.y;  // [0, cp): fwd of step i; [cp, 2cp): dkdv of step i - cp
  const bool is_fwd = list < cp;
  const int i = is_fwd ? list : list - cp;
  const int kind = sw[SW_KIND + i];
  const int32_t* off = tabp + (is_fwd ? L.fwd_off : L.dkdv_off) + (int64_t)i * (B + 1);
  const int total = off[B];
  const int64_t cap = is_fwd ? L.fwd_cap : L.dkdv_cap;
  int32_t* items = tabp + (is_fwd ? L.fwd_tiles : L.dkdv_tiles) + (int64_t)i * cap * 2;
  int32_t* keys = tabp + (is_fwd ? L.fwd_keys : L.dkdv_keys) + (int64_t)i * cap * 2;
  const int32_t* st = tabp + L.steps + (int64_t)i * 4 * B;
  const int32_t* cup = tabp + L.cup;
  for (int f = blockIdx.x * blockDim.x + threadIdx.x; f < total; f += gridDim.x * blockDim.x) {
    int b = upper_idx(off, B, f);
    while (b < B - 1 && off[b + 1] <= f) ++b;
    while (b > 0 && off[b] > f) --b;
    const int n_b = off[b + 1] - off[b];
    const int t = n_b - 1 - (f - off[b]);  // last tile first within a sequence
    const int q_len = st[B + b], kv_len = st[3 * B + b];
    long long work;
    if (is_fwd) {
      int rows = min(FWD_BM, q_len - t * FWD_BM);
      int keys_n = kind == 0 ? min(kv_len, (t + 1) * FWD_BM) : kv_len;
      work = (long long)rows * keys_n;
      if (i == 0) {
        // step 0's items are also the blocks of the single-launch forward,
        // where each block runs the key tiles of every step its rows take
        // part in: the sum of those steps' keys, for the whole block
        const int q0 = t * FWD_BM, q1 = q0 + rows;
        long long keys_all = 0;
        for (int j = 0; j < cp; ++j) {
          const int32_t* sj = tabp + L.steps + (int64_t)j * 4 * B;
          const int rlo = sj[b] - st[b], rhi = rlo + sj[B + b];
          if (max(q0, rlo) >= min(q1, rhi)) continue;
          const int kl = sj[3 * B + b];
          keys_all += sw[SW_KIND + j] == 0 ? min(kl, q1) : kl;
        }
        work = (long long)FWD_BM * keys_all;
      }
    } else {
      int nk = clampi(kv_len - t * DKDV_BN, 0, DKDV_BN);
      int nq = kind == 0 ? max(0, q_len - t * DKDV_BN) : q_len;
      work = (long long)nk * nq;
      (void)cup;
    }
    items[2 * f] = b;
    items[2 * f + 1] = t;
    keys[f] = (int)min(work >> 4, (long long)0x7fffffff) + 1;
  }
}

// Heaviest-first ordering of one work list (bitonic sort in LDS).
__global__ void __launch_bounds__(1024) meta_sort_kernel(int32_t* __restrict__ tabp, MetaLayout L, int B, int cp) {
  __shared__ unsigned long long sv[SORT_CAP];
  const int32_t* sw = tabp + L.summary;
  if (sw[SW_ERR]) return;
  const int list = blockIdx.x;
  const bool is_fwd = list < cp;
  const int i = is_fwd ? list : list - cp;
  const int total = sw[(is_fwd ? SW_TILES_FWD : SW_TILES_DKDV) + i];
  if (total <= 1 || total > SORT_CAP) return;
  const int64_t cap = is_fwd ? L.fwd_cap : L.dkdv_cap;
  int32_t* items = tabp + (is_fwd ? L.fwd_tiles : L.dkdv_tiles) + (int64_t)i * cap * 2;
  int32_t* keys = tabp + (is_fwd ? L.fwd_keys : L.dkdv_keys) + (int64_t)i * cap * 2;
  int n = 1;
  while (n < total) n <<= 1;
  for (int p = threadIdx.x; p < n; p += blockDim.x) {
    sv[p] = p < total ? ((unsigned long long)(unsigned)keys[p] << 32) | (0xffffffffu - (unsigned)p) : 0ull;
  }
  __syncthreads();
  // descending bitonic sort
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int p = threadIdx.x; p < n; p += blockDim.x) {
        int q = p ^ j;
        if (q > p) {
          unsigned long long a = sv[p], b = sv[q];
          bool desc = (p & k) == 0;
          if (desc ? (a < b) : (a > b)) {
            sv[p] = b;
            sv[q] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // gather through the key scratch (2 ints per item), then copy back
  for (int p = threadIdx.x; p < total; p += blockDim.x) {
    unsigned idx = 0xffffffffu - (unsigned)(sv[p] & 0xffffffffull);
    keys[2 * p] = items[2 * idx];
    keys[2 * p + 1] = items[2 * idx + 1];
  }
  __syncthreads();
  __threadfence_block();
  for (int p = threadIdx.x; p < 2 * total; p += blockDim.x) items[p] = keys[p];
}

// Gather rank `shard`'s rows out of a global packed tensor (16-byte units).
__global__ void shard_gather_kernel(const int32_t* __restrict__ tabp, MetaLayout L, int B, int cp, int shard,
                                    const uint4* __restrict__ src, uint4* __restrict__ dst, int units_per_row,
                                    int t_local) {
  const int32_t* cupl = tabp + L.cupl;
  const int32_t* chunk = tabp + L.chunk;
  const int32_t* cup = tabp + L.cup;
  const long long n = (long long)t_local * units_per_row;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n; e += (long long)gridDim.x * blockDim.x) {
    const int t = (int)(e / units_per_row);
    const int u = (int)(e - (long long)t * units_per_row);
    int b = upper_idx(cupl, B, t);
    if (b >= B) b = B - 1;
    while (b > 0 && cupl[b] == cupl[b + 1]) --b;
    const int o = t - cupl[b];
    const int c = chunk[b];
    const int k = o < c ? shard : 2 * cp - 1 - shard;
    const long long g = (long long)cup[b] + (long long)k * c + (o < c ? o : o - c);
    dst[e] = src[g * units_per_row + u];
  }
}

}  // namespace cpattn

using namespace cpattn;

static std::string describe_meta_error(int e) {
  std::string s;
  if (e & ME_START) s += "cu_seqlens / cu_seqlens_padded must start at 0; ";
  if (e & ME_CU_ORDER) s += "cu_seqlens must be non-decreasing; ";
  if (e & ME_CUP_ORDER) s += "cu_seqlens_padded must be non-decreasing; ";
  if (e & ME_LEN) s += "a valid length exceeds its padded length; ";
  if (e & ME_DIV) s += "a padded sequence length is not divisible by 2*cp_size; ";
  if (e & ME_ALLOC) s += "t_alloc is smaller than cu_seqlens_padded[B]/cp_size; ";
  if (e & ME_RANGE) s += "packed length too large for 31-bit row indices; ";
  if (e & ME_HINT) s += "pad_hint contradicts the values of cu_seqlens / cu_seqlens_padded; ";
  return s;
}

// Pinned landing buffer of the summary: one per calling thread and device,
// allocated on first use and kept until the process ends (the summary is read
// within the call that copies it, so one buffer serves every call).
static cp_attn_status summary_buffer(int device, int32_t** out) {
  static thread_local int32_t* buf[64] = {};
  if (device < 0 || device >= 64) return fail(CP_ATTN_ERR_INVALID_ARG, "device index out of range");
  if (!buf[device]) {
    cp_attn_status rc = hip_check(hipHostMalloc((void**)&buf[device], SW_COUNT * sizeof(int32_t), hipHostMallocDefault),
                                  "hipHostMalloc(summary)");
    if (rc != CP_ATTN_OK) {
      buf[device] = nullptr;
      return rc;
    }
  }
  *out = buf[device];
  return CP_ATTN_OK;
}

// Device table buffers. A freed handle's buffer (the free synchronises the
// device first, so no queued kernel still reads it) goes back to a free list
// of its device, and the next handle on that device whose tables fit takes
// it: steady-state metadata builds call no hipMalloc. At most POOL_MAX
// buffers per device are kept, until the process ends.
namespace {
constexpr size_t POOL_MAX = 64;
struct TabPool {
  std::mutex mu;
  std::vector<std::pair<int32_t*, size_t>> free;
};
TabPool g_pool[64];
}  // namespace

static cp_attn_status tab_alloc(int device, size_t bytes, int32_t** p, size_t* got) {
  bytes = (bytes + 65535) & ~size_t(65535);
  if (device >= 0 && device < 64) {
    TabPool& tp = g_pool[device];
    std::lock_guard<std::mutex> lk(tp.mu);
    int best = -1;
    for (int i = 0; i < (int)tp.free.size(); ++i)
      if (tp.free[i].second >= bytes && tp.free[i].second <= 4 * bytes &&
          (best < 0 || tp.free[i].second < tp.free[best].second))
        best = i;
    if (best >= 0) {
      *p = tp.free[best].first;
      *got = tp.free[best].second;
      tp.free.erase(tp.free.begin() + best);
      return CP_ATTN_OK;
    }
  }
  *got = bytes;
  return hip_check(hipMalloc(p, bytes), "hipMalloc(meta)");
}

static void tab_release(int device, int32_t* p, size_t bytes) {
  if (device >= 0 && device < 64) {
    TabPool& tp = g_pool[device];
    std::lock_guard<std::mutex> lk(tp.mu);
    if (tp.free.size() < POOL_MAX) {
      tp.free.emplace_back(p, bytes);
      return;
    }
  }
  hipFree(p);
}

static cp_attn_status check_meta_args(const int32_t* cu, int B, int cp_size, int cp_rank, int pad_hint,
                                      int64_t t_alloc, cp_attn_meta** out) {
  if (!out) return fail(CP_ATTN_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!cu) return fail(CP_ATTN_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if (B < 1) return fail(CP_ATTN_ERR_INVALID_ARG, "B must be >= 1");
  if (cp_size < 1 || cp_size > CP_ATTN_MAX_CP) return fail(CP_ATTN_ERR_UNSUPPORTED, "cp_size must be in [1, 16]");
  if (cp_rank < 0 || cp_rank >= cp_size) return fail(CP_ATTN_ERR_INVALID_ARG, "cp_rank out of range");
  if (pad_hint < -1 || pad_hint > 1) return fail(CP_ATTN_ERR_INVALID_ARG, "pad_hint must be -1, 0 or 1");
  if (t_alloc < 0 || t_alloc >= (1ll << 30)) return fail(CP_ATTN_ERR_INVALID_ARG, "t_alloc out of range");
  return CP_ATTN_OK;
}

// A handle with its device tables, and the metadata kernels launched on st
// (the tables kernel reading its inputs from src).
template <class Src>
static cp_attn_status launch_meta(const Src& src, int B, int cp_size, int cp_rank, int pad_hint, int64_t t_alloc,
                                  hipStream_t st, cp_attn_meta** out) {
  cp_attn_meta* m = new cp_attn_meta();
  std::memset(&m->sum, 0, sizeof(m->sum));
  m->B = B;
  m->cp = cp_size;
  m->rank = cp_rank;
  m->pad_hint = pad_hint;
  m->t_alloc = t_alloc;
  m->lay = make_layout(B, cp_size, t_alloc);
  m->d_tab = nullptr;
  m->sum.B = B;
  m->sum.cp_size = cp_size;
  m->sum.cp_rank = cp_rank;
  m->sum.t_alloc = t_alloc;
  cp_attn_status rc;
  if ((rc = hip_check(hipGetDevice(&m->device), "hipGetDevice")) != CP_ATTN_OK) { delete m; return rc; }
  m->tab_bytes = 0;
  if ((rc = tab_alloc(m->device, m->lay.total * sizeof(int32_t), &m->d_tab, &m->tab_bytes)) != CP_ATTN_OK) {
    delete m;
    return rc;
  }
  const MetaLayout& L = m->lay;
  hipLaunchKernelGGL(meta_tables_kernel<Src>, dim3(1), dim3(256), 0, st, src, B, cp_size, cp_rank, pad_hint,
                     (long long)t_alloc, m->d_tab, L);
  {
    long long blocks = std::min<long long>((t_alloc + 255) / 256, 4096);
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(meta_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, m->d_tab, L, B, cp_size, cp_rank,
                       (long long)t_alloc);
  }
  {
    long long cap = std::max(L.fwd_cap, L.dkdv_cap);
    unsigned bx = (unsigned)std::min<long long>((cap + 255) / 256, 1024);
    hipLaunchKernelGGL(meta_tiles_kernel, dim3(bx, 2 * cp_size), dim3(256), 0, st, m->d_tab, L, B, cp_size);
  }
  hipLaunchKernelGGL(meta_sort_kernel, dim3(2 * cp_size), dim3(1024), 0, st, m->d_tab, L, B, cp_size);
  if ((rc = hip_check(hipGetLastError(), "metadata kernel launch")) != CP_ATTN_OK) {
    cp_attn_meta_free(m);
    return rc;
  }
  *out = m;
  return CP_ATTN_OK;
}

// The summary and the validation word from host copies of the inputs: the
// same arithmetic as the tables kernel's (chunk sizes P_b / (2 CP), valid
// rows per chunk, step kinds and sources, work-item counts per step).
static int host_summary(const int32_t* cu, const int32_t* cup_in, int B, int cp, int rank, int hint, int64_t t_alloc,
                        cp_attn_summary* s) {
  const int32_t* cup = cup_in ? cup_in : cu;
  auto cv = [](int L, int c, int k) { return std::min(std::max(L - k * c, 0), c); };
  const int two_cp = 2 * cp;
  int err = 0, pad = 0;
  if (cu[0] != 0 || cup[0] != 0) err |= ME_START;
  for (int b = 0; b <= B; ++b)
    if (cu[b] != cup[b]) pad = 1;
  for (int i = 0; i < cp; ++i) {
    const int src = ((rank - i) % cp + cp) % cp;
    s->step_src[i] = src;
    s->step_kind[i] = i == 0 ? 0 : (src < rank ? 1 : 2);
  }
  int64_t valid = 0;
  for (int b = 0; b < B; ++b) {
    int Lb = cu[b + 1] - cu[b], Pb = cup[b + 1] - cup[b];
    if (Lb < 0) err |= ME_CU_ORDER;
    if (Pb < 0) err |= ME_CUP_ORDER;
    if (Lb > Pb) err |= ME_LEN;
    if (Pb >= 0 && Pb % two_cp != 0) err |= ME_DIV;
    if (Pb < 0) Pb = 0;
    Lb = std::min(std::max(Lb, 0), Pb);
    const int c = Pb / two_cp;
    const int fr = cv(Lb, c, rank), sr = cv(Lb, c, two_cp - 1 - rank);
    valid += fr + sr;
    for (int i = 0; i < cp; ++i) {
      const int q_len = s->step_kind[i] == 2 ? sr : fr + sr;
      s->tiles_fwd[i] += (q_len + FWD_BM - 1) / FWD_BM;
      s->tiles_dkdv[i] += (Pb / cp + DKDV_BN - 1) / DKDV_BN;
    }
  }
  const int64_t tl = (int64_t)cup[B] / cp;
  if (tl > t_alloc) err |= ME_ALLOC;
  if (tl >= (1ll << 30)) err |= ME_RANGE;
  if (hint >= 0 && hint != pad) err |= ME_HINT;
  s->pad_between_seqs = pad;
  s->t_local = (int32_t)tl;
  s->has_tail = t_alloc > tl ? 1 : 0;
  s->valid_rows = valid;
  return err;
}

extern "C" {

const char* cp_attn_last_error(void) { return g_last_error.c_str(); }

cp_attn_status cp_attn_rank_metadata(const int32_t* cu_seqlens, const int32_t* cu_seqlens_padded, int32_t B,
                                     int32_t cp_size, int32_t cp_rank, int32_t pad_hint, int64_t t_alloc,
                                     void* stream, cp_attn_meta** out) {
  set_error("");
  cp_attn_status rc = check_meta_args(cu_seqlens, B, cp_size, cp_rank, pad_hint, t_alloc, out);
  if (rc != CP_ATTN_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  int32_t* h_sum = nullptr;
  int device = 0;
  if ((rc = hip_check(hipGetDevice(&device), "hipGetDevice")) != CP_ATTN_OK) return rc;
  if ((rc = summary_buffer(device, &h_sum)) != CP_ATTN_OK) return rc;
  cp_attn_meta* m = nullptr;
  if ((rc = launch_meta(DevSeqlens{cu_seqlens, cu_seqlens_padded}, B, cp_size, cp_rank, pad_hint, t_alloc, st, &m)) !=
      CP_ATTN_OK)
    return rc;
  const MetaLayout& L = m->lay;
  if ((rc = hip_check(hipMemcpyAsync(h_sum, m->d_tab + L.summary, SW_COUNT * sizeof(int32_t),
                                     hipMemcpyDeviceToHost, st),
                      "hipMemcpyAsync(summary)")) != CP_ATTN_OK) {
    cp_attn_meta_free(m);
    return rc;
  }
  if ((rc = hip_check(hipStreamSynchronize(st), "hipStreamSynchronize(metadata)")) != CP_ATTN_OK) {
    cp_attn_meta_free(m);
    return rc;
  }
  const int32_t* sw = h_sum;
  const int err = sw[SW_ERR];
  if (err) {
    cp_attn_meta_free(m);
    return fail(err == ME_HINT ? CP_ATTN_ERR_HINT_MISMATCH : CP_ATTN_ERR_INVALID_ARG, describe_meta_error(err));
  }
  cp_attn_summary& s = m->sum;
  s.pad_between_seqs = sw[SW_PAD];
  s.t_local = sw[SW_TLOCAL];
  s.has_tail = sw[SW_HAS_TAIL];
  s.valid_rows = sw[SW_VALID_ROWS];
  for (int i = 0; i < cp_size; ++i) {
    s.step_kind[i] = sw[SW_KIND + i];
    s.step_src[i] = sw[SW_SRC + i];
    s.tiles_fwd[i] = sw[SW_TILES_FWD + i];
    s.tiles_dkdv[i] = sw[SW_TILES_DKDV + i];
  }
  *out = m;
  return CP_ATTN_OK;
}

cp_attn_status cp_attn_rank_metadata_host(const int32_t* cu_seqlens, const int32_t* cu_seqlens_padded, int32_t B,
                                          int32_t cp_size, int32_t cp_rank, int32_t pad_hint, int64_t t_alloc,
                                          void* stream, cp_attn_meta** out) {
  set_error("");
  cp_attn_status rc = check_meta_args(cu_seqlens, B, cp_size, cp_rank, pad_hint, t_alloc, out);
  if (rc != CP_ATTN_OK) return rc;
  if (B > CP_ATTN_HOST_META_MAX_B)
    return fail(CP_ATTN_ERR_UNSUPPORTED, "more sequences than the host path carries; use cp_attn_rank_metadata");
  cp_attn_summary s{};
  const int err = host_summary(cu_seqlens, cu_seqlens_padded, B, cp_size, cp_rank, pad_hint, t_alloc, &s);
  if (err) return fail(err == ME_HINT ? CP_ATTN_ERR_HINT_MISMATCH : CP_ATTN_ERR_INVALID_ARG, describe_meta_error(err));
  ArgSeqlens vals;
  for (int b = 0; b <= B; ++b) {
    vals.cu[b] = cu_seqlens[b];
    vals.cup[b] = cu_seqlens_padded ? cu_seqlens_padded[b] : cu_seqlens[b];
  }
  cp_attn_meta* m = nullptr;
  if ((rc = launch_meta(vals, B, cp_size, cp_rank, pad_hint, t_alloc, (hipStream_t)stream, &m)) != CP_ATTN_OK)
    return rc;
  const cp_attn_summary keep = m->sum;  // B, ring and t_alloc, filled by launch_meta
  m->sum = s;
  m->sum.B = keep.B;
  m->sum.cp_size = keep.cp_size;
  m->sum.cp_rank = keep.cp_rank;
  m->sum.t_alloc = keep.t_alloc;
  *out = m;
  return CP_ATTN_OK;
}

cp_attn_status cp_attn_meta_summary(const cp_attn_meta* m, cp_attn_summary* out) {
  if (!m || !out) return fail(CP_ATTN_ERR_INVALID_ARG, "NULL argument");
  *out = m->sum;
  return CP_ATTN_OK;
}

cp_attn_status cp_attn_meta_export(const cp_attn_meta* m, int32_t* host_buf, size_t n, size_t* n_needed) {
  if (!m) return fail(CP_ATTN_ERR_INVALID_ARG, "meta is NULL");
  const int B = m->B, cp = m->cp;
  const size_t need = 8 + (size_t)B + 2 * (size_t)(B + 1) + 3 * (size_t)cp * (B + 1) + (size_t)cp * (2 + 4 * (size_t)B);
  if (n_needed) *n_needed = need;
  if (!host_buf) return CP_ATTN_OK;
  if (n < need) return fail(CP_ATTN_ERR_INVALID_ARG, "export buffer too small");
  int cur = 0;
  hipGetDevice(&cur);
  if (cur != m->device) hipSetDevice(m->device);
  cp_attn_status rc = hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize(export)");
  if (rc != CP_ATTN_OK) return rc;
  const MetaLayout& L = m->lay;
  int32_t* h = new int32_t[L.total];
  rc = hip_check(hipMemcpy(h, m->d_tab, L.total * sizeof(int32_t), hipMemcpyDeviceToHost), "hipMemcpy(export)");
  if (cur != m->device) hipSetDevice(cur);
  if (rc != CP_ATTN_OK) { delete[] h; return rc; }
  size_t o = 0;
  const cp_attn_summary& s = m->sum;
  int32_t hdr[8] = {B, cp, m->rank, s.pad_between_seqs, s.t_local, s.has_tail, cp, 0};
  for (int k = 0; k < 8; ++k) host_buf[o++] = hdr[k];
  for (int b = 0; b < B; ++b) host_buf[o++] = h[L.chunk + b];
  for (int b = 0; b <= B; ++b) host_buf[o++] = h[L.cupl + b];
  for (int b = 0; b <= B; ++b) host_buf[o++] = h[L.cuph + b];
  for (int sh = 0; sh < cp; ++sh) {
    for (int b = 0; b <= B; ++b) host_buf[o++] = h[L.cu_full + (int64_t)sh * (B + 1) + b];
    for (int b = 0; b <= B; ++b) host_buf[o++] = h[L.cu_first + (int64_t)sh * (B + 1) + b];
    for (int b = 0; b <= B; ++b) host_buf[o++] = h[L.cu_second + (int64_t)sh * (B + 1) + b];
  }
  for (int i = 0; i < cp; ++i) {
    host_buf[o++] = s.step_kind[i];
    host_buf[o++] = s.step_src[i];
    for (int k = 0; k < 4 * B; ++k) host_buf[o++] = h[L.steps + (int64_t)i * 4 * B + k];
  }
  delete[] h;
  return CP_ATTN_OK;
}

void cp_attn_meta_free(cp_attn_meta* m) {
  if (!m) return;
  int cur = 0;
  hipGetDevice(&cur);
  if (cur != m->device) hipSetDevice(m->device);
  if (m->d_tab) {
    hipDeviceSynchronize();
    tab_release(m->device, m->d_tab, m->tab_bytes);
  }
  if (cur != m->device) hipSetDevice(cur);
  delete m;
}

cp_attn_status cp_attn_shard_gather(const cp_attn_meta* m, int32_t shard, const void* global, void* local,
                                    size_t row_bytes, void* stream) {
  if (!m || !global || !local) return fail(CP_ATTN_ERR_INVALID_ARG, "NULL argument");
  if (shard < 0 || shard >= m->cp) return fail(CP_ATTN_ERR_INVALID_ARG, "shard out of range");
  if (row_bytes == 0 || row_bytes % 16 != 0 || row_bytes > (1u << 30))
    return fail(CP_ATTN_ERR_INVALID_ARG, "row_bytes must be a positive multiple of 16");
  if (((uintptr_t)global | (uintptr_t)local) & 15) return fail(CP_ATTN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const int tl = m->sum.t_local;
  if (tl == 0) return CP_ATTN_OK;
  const int upr = (int)(row_bytes / 16);
  long long n = (long long)tl * upr;
  unsigned blocks = (unsigned)std::min<long long>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(shard_gather_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, m->d_tab, m->lay, m->B,
                     m->cp, shard, (const uint4*)global, (uint4*)local, upr, tl);
  return hip_check(hipGetLastError(), "shard_gather launch");
}

}  // extern "C"
