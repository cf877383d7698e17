// Forward of one CP rank's share: flash-style MFMA kernels over the ring
// steps, with the log-sum-exp merge of the steps' partials.
//
// "thd format is not supported with hierarchical CP implementation yet": the
// P2P ring delivers one KV shard per step and long sequences keep the ring's
// exchange under compute. What each step computes follows from the
// load-balanced pairing of chunks r and 2*CP-1-r ("Hybrid / Hierarchical
// Context Parallel Skill", "Enablement"): step 0 is causal on local rows;
// a shard from an earlier rank is seen in full by all query rows but only
// through its first chunk; a shard from a later rank is seen in full by the
// second query chunk only. The merge is the exact softmax identity
//   lse = log(e^la + e^lb),  O = e^(la-lse) Oa + e^(lb-lse) Ob.
// Long shares run one launch per step, each folding its partial into an fp32
// accumulator in its epilogue by that identity; short shares run every step
// in one launch whose blocks carry the online softmax's running max and sum
// across the steps (the same identity applied key tile by key tile), so no
// partial leaves the registers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "internal.h"
#include "kern_common.h"

namespace cpattn {

struct FwdParams {
  const uint16_t* q;
  const int32_t* steps;  // every step's sequence tables: [step][q_start, q_len, kv_start, kv_len][B]
  int B;
  int hq, group;
  long long ld_q, ld_kv;  // elements per row
  float scale, c_log2;    // softmax scale, scale * log2(e)
  long long ld_o, ld_lse;
  // epilogue: 1 = fold the step's normalised partial into the accumulator
  // (o, lse) through the log-sum-exp; 2 = fold it and write the result as
  // the bf16 output and final LSE instead (the fused launch writes those
  // itself). acc_first /
  // acc_second: whether the accumulator already holds rows of the first /
  // second chunk (earlier steps covered them).
  int mode, acc_first, acc_second;
  const int32_t* rowflags;
  uint16_t* out;
  float* lse_out;
  long long ld_lse_out;
};

// The ring steps of one launch: blocks [off[j], off[j + 1]) compute ring step
// step[j] (kind kind[j]) against K / V shard k[j] / v[j], over its work items
// items[j], folding into the running accumulator o[j] (fp32 [rows, hq, D])
// and lse[j] (fp32 [hq, ld_lse]); the fused launch runs every entry in each
// block, over entry 0's work items, and needs no accumulator.
struct FwdSteps {
  const uint16_t* k[CP_ATTN_MAX_CP];
  const uint16_t* v[CP_ATTN_MAX_CP];
  const int32_t* items[CP_ATTN_MAX_CP];
  float* o[CP_ATTN_MAX_CP];
  float* lse[CP_ATTN_MAX_CP];
  int step[CP_ATTN_MAX_CP];
  int kind[CP_ATTN_MAX_CP];
  int off[CP_ATTN_MAX_CP + 1];
  int n;
};

// A step's normalised partial for one lane's query row (local row t): mode 1
// folds it into the accumulator through the log-sum-exp, mode 2 folds it and
// writes the bf16 output and the final LSE instead:
//   out = (e^(la-m) out_a + e^(lb-m) out_b) / (e^(la-m) + e^(lb-m)),
//   lse = m + log of that sum, m = max(la, lb).
template <int D>
__device__ __forceinline__ void step_epilogue(const FwdParams& p, float* o_part, float* l_part, int t, int head, int g,
                                              const f32x16_t (&o)[D / 32], float m_run, float lt) {
  constexpr int NMD = D / 32;
  float inv, lse;
  if (lt > 0.f) {
    inv = 1.f / lt;
    lse = m_run * p.scale + __logf(lt);
  } else {
    inv = 0.f;
    lse = NEG_INF_F;
  }
  float* orow = o_part + (long long)t * p.ld_o + head * D + g * 4;
  float* lrow = l_part + (long long)head * p.ld_lse + t;
  const bool has = (p.rowflags[t] & RF_SECOND) ? p.acc_second : p.acc_first;
  const float la = has ? *lrow : NEG_INF_F;
  const float mx = fmaxf(la, lse);
  float wa = 0.f, wb = 0.f, lm = NEG_INF_F;
  if (mx != NEG_INF_F) {
    wa = __expf(la - mx);
    wb = __expf(lse - mx);
    const float ssum = wa + wb;
    lm = mx + __logf(ssum);
    const float r = 1.f / ssum;
    wa *= r;
    wb *= r * inv;
  }
  uint16_t* out_row = p.out + (long long)t * p.ld_o + head * D + g * 4;
#pragma unroll
  for (int md = 0; md < NMD; ++md)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
      if (has) a = *reinterpret_cast<const float4*>(orow + md * 32 + jj * 8);
      const float4 val = make_float4(wa * a.x + wb * o[md][4 * jj], wa * a.y + wb * o[md][4 * jj + 1],
                                     wa * a.z + wb * o[md][4 * jj + 2], wa * a.w + wb * o[md][4 * jj + 3]);
      if (p.mode == 1) {
        *reinterpret_cast<float4*>(orow + md * 32 + jj * 8) = val;
      } else {
        uint2 pk;
        pk.x = pack2_bf16(val.x, val.y);
        pk.y = pack2_bf16(val.z, val.w);
        *reinterpret_cast<uint2*>(out_row + md * 32 + jj * 8) = pk;
      }
    }
  if (g == 0) {
    if (p.mode == 1)
      *lrow = lm;
    else
      p.lse_out[(long long)head * p.ld_lse_out + t] = lm;
  }
}

// One block = NWAVES wavefronts (FWD_BM query rows) of one head; each wavefront owns
// 32 query rows. K and V tiles of BN rows (64; 32 in the fused launch) are
// copied straight from global memory into padded LDS tiles (buffer loads
// with the lds modifier, no register staging), double-buffered. Scores are computed transposed
// (S^T = K Q^T, K rows as the A operand) so each lane owns one query row: the
// online softmax needs one cross-lane max per tile, and O^T = V^T P^T takes
// V^T through transposing LDS reads and keeps per-lane row scaling. Keys past
// the step's key range read as zeros (buffer range check) and are masked.
// Rescaling is lazy: the running max only moves when a tile's max exceeds it
// by more than 2^8 in exp2 units.
// FUSED = false: the block computes one ring step (entry si of the list, its
// rows relative to that step's query range) and its epilogue writes or folds
// that step's normalised partial (p.mode). FUSED = true: the block's rows come
// from entry 0's work items (the causal step, which covers every valid row of
// its sequence slot) and it runs through every entry's key tiles in turn, so
// the online softmax carries the running max and sum from one ring step to
// the next and the log-sum-exp merge of the steps happens in registers; the
// epilogue writes the bf16 output and the final LSE. Rows outside an entry's
// query range take no part in it (masked).
template <int D, bool FUSED, int BN>
__global__ void __launch_bounds__(BLOCK_THREADS, BN == 32 ? 3 : 8 / NWAVES) fwd_step_kernel(FwdParams p, FwdSteps st) {
  constexpr int BM = FWD_BM;
  constexpr int NKK = D / 16;
  constexpr int NMD = D / 32;
  constexpr int MB = BN / 32, KK2 = BN / 16;  // 32-key score blocks, 16-key P V slices per tile
  using KCopy = TileCopy<D, false, BN, NWAVES>;
  using VCopy = TileCopy<D, true, BN, NWAVES>;
  __shared__ __attribute__((aligned(1024))) uint16_t Ks[2][KCopy::BYTES / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs[2][VCopy::BYTES / 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index (uniform)
  // this block's entry of the list (every block of one entry shares it)
  int si = 0;
  if constexpr (!FUSED) {
    while (si + 1 < st.n && (int)blockIdx.x >= st.off[si + 1]) ++si;
    si = __builtin_amdgcn_readfirstlane(si);
  }
  int item, head;
  map_block((int)blockIdx.x - st.off[si], p.hq, item, head);
  const int sb = st.items[si][2 * item], tile = st.items[si][2 * item + 1];
  // entry j's sequence tables: [step][q_start, q_len, kv_start, kv_len][B].
  // FUSED: every entry's four values are read once into LDS, so moving on
  // to the next entry mid-loop reads LDS and does not wait for the tile
  // copies in flight (a global read would: the load counter retires in
  // order)
  __shared__ int ent_tab[FUSED ? 4 * CP_ATTN_MAX_CP : 1];
  if constexpr (FUSED) {
    for (int j = 0; j < st.n; ++j)
      if (tid < 4) ent_tab[4 * j + tid] = p.steps[((long long)st.step[j] * 4 + tid) * p.B + sb];
    __syncthreads();
  }
  auto tab = [&](int j, int f) {
    if constexpr (FUSED)
      return ent_tab[4 * j + f];
    else
      return p.steps[((long long)st.step[j] * 4 + f) * p.B + sb];
  };
  const int qs = tab(si, 0), ql = tab(si, 1);  // the block's rows are relative to qs
  const int q0 = tile * BM;
  const int nq = min(BM, ql - q0);
  const int kvh = head / p.group;
  const float c = p.c_log2;

  const int qrow = q0 + w * 32 + l32;  // relative to qs
  bf16x8_t qf[NKK];
  {
    const bool ok = qrow < ql;
    const uint16_t* src = p.q + (long long)(qs + (ok ? qrow : 0)) * p.ld_q + head * D + g * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 u = ok ? *reinterpret_cast<const uint4*>(src + kk * 16) : make_uint4(0, 0, 0, 0);
      qf[kk] = as_bf16x8(u);
    }
  }

  f32x16_t o[NMD];
#pragma unroll
  for (int md = 0; md < NMD; ++md) o[md] = zero16();
  float m_run = NEG_INF_F, l_run = 0.f;

  const int ldb = (int)(p.ld_kv * 2);
  // A position in the block's sequence of key tiles: entry j, key tile kt of
  // its nt, with the entry's query rows [rlo, rhi) (relative to qs), keys,
  // mask kind, and where its K and V rows start (kb, vb) with the byte end
  // of its key range (end32; -1 when a tile offset could pass 2^31, which
  // then takes 64-bit arithmetic). Everything but kt is set once per entry,
  // so a tile's copy only adds its offset.
  struct Cur {
    int j, kt, nt, rlo, rhi, kl, causal, end32;
    const uint16_t* kb;
    const uint16_t* vb;
  };
  auto at = [&](int j) {
    Cur u;
    u.j = j;
    u.kt = 0;
    u.rlo = FUSED ? tab(j, 0) - qs : 0;
    u.rhi = FUSED ? u.rlo + tab(j, 1) : ql;
    u.kl = tab(j, 3);
    u.causal = st.kind[j] == 0;
    const long long row0 = (long long)tab(j, 2) * p.ld_kv + kvh * D;
    u.kb = st.k[j] + row0;
    u.vb = st.v[j] + row0;
    const long long end = (long long)u.kl * ldb;
    u.end32 = end <= 0x7fffffffLL ? (int)end : -1;
    const int lo = max(q0, u.rlo), hi = min(q0 + nq, u.rhi);
    const int n_keys = hi <= lo ? 0 : (u.causal ? min(u.kl, q0 + nq) : u.kl);
    u.nt = (n_keys + BN - 1) / BN;
    return u;
  };
  // on to the next key tile (FUSED: possibly the first of a later entry);
  // false past the last
  auto advance = [&](Cur& u) {
    if (++u.kt < u.nt) return true;
    if constexpr (FUSED) {
      while (u.j + 1 < st.n) {
        u = at(u.j + 1);
        if (u.nt > 0) return true;
      }
    }
    return false;
  };
  KCopy kc;
  VCopy vc;
  kc.init(ldb, w, lane);
  vc.init(ldb, w, lane);
  auto issue = [&](const Cur& u, int buf) {
    if (u.end32 >= 0) {
      const int off = u.kt * (BN * ldb);  // below end32, so below 2^31
      kc.copy(rsrc_from32(u.kb, off, u.end32), Ks[buf], w);
      vc.copy(rsrc_from32(u.vb, off, u.end32), Vs[buf], w);
    } else {
      const long long off = (long long)u.kt * BN * ldb, end = (long long)u.kl * ldb;
      kc.copy(rsrc_from(u.kb, off, end), Ks[buf], w);
      vc.copy(rsrc_from(u.vb, off, end), Vs[buf], w);
    }
  };

  const float lazy_thr = 8.0f / c;  // 2^8 headroom, in raw score units
  // first half of a key tile: scores, V fragments, softmax, P packed to
  // bf16; masking runs only on a wavefront's last tiles (keys past the
  // range, or at the causal step keys after its first row) and, fused, on
  // the tiles of entries whose query range splits the wavefront's rows
  auto key_tile = [&](const Cur& u, int buf, bool masked, bf16x8_t (&pb)[KK2], bf16x8_t (&vf)[KK2][NMD]) {
    const int k0 = u.kt * BN;
    f32x16_t s[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) s[mb] = zero16();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        s[mb] = mfma32x32x16(lds_read_row<D>(Ks[buf], mb * 32 + l32, 2 * kk + g), qf[kk], s[mb]);
    }
    // all V fragments of the tile are read now, so the LDS latency hides
    // behind the softmax instead of stalling the P V products (the
    // scheduling fence keeps the compiler from sinking the reads again)
#pragma unroll
    for (int kk2 = 0; kk2 < KK2; ++kk2)
#pragma unroll
      for (int md = 0; md < NMD; ++md) vf[kk2][md] = lds_read_tr<D, true>(Vs[buf], kk2 * 16, md * 32, lane);
    __builtin_amdgcn_sched_barrier(0);
    if (masked) {
      // a real branch (kept out of if-conversion), taken on few tiles
      __asm__ volatile("" ::: "memory");
      // element (mb, j) holds key k0 + 4 g + off, off = 32 mb + 8 (j / 4) +
      // j % 4; it counts when the key is below lim (the range end, and at
      // the causal step the row's own position + 1; nothing for rows outside
      // the entry): one compare of off against a per-lane bound
      const bool row_in = !FUSED || (qrow >= u.rlo && qrow < u.rhi);
      const int lim = !row_in ? -(1 << 20) : (u.causal ? min(u.kl, qrow + 1) : u.kl);
      const int r = lim - 1 - (k0 + 4 * g);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[mb][j] = (r - (mb * 32 + (j >> 2) * 8 + (j & 3)) >= 0) ? s[mb][j] : NEG_INF_F;
    }
    float mx = NEG_INF_F;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[mb][j]);
    mx = max_halves(mx);
    const bool need = mx > m_run + lazy_thr;
    if (__any(need)) {
      const float alpha = need ? fast_exp2((m_run - mx) * c) : 1.f;
      if (need) m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int md = 0; md < NMD; ++md)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[md][j] *= alpha;
    }
    const float base = (m_run == NEG_INF_F) ? 0.f : m_run * c;
    float lsum = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pv = fast_exp2(fmaf(s[mb][j], c, -base));
        s[mb][j] = pv;
        lsum += pv;
      }
    l_run += lsum;
#pragma unroll
    for (int kk2 = 0; kk2 < KK2; ++kk2) pb[kk2] = pack8_bf16(s[kk2 >> 1], 8 * (kk2 & 1));
  };
  // second half: O += P V from registers
  auto pv_tile = [&](const bf16x8_t (&pb)[KK2], const bf16x8_t (&vf)[KK2][NMD]) {
#pragma unroll
    for (int kk2 = 0; kk2 < KK2; ++kk2)
#pragma unroll
      for (int md = 0; md < NMD; ++md) o[md] = mfma32x32x16(vf[kk2][md], pb[kk2], o[md]);
  };

  // Tile it's buffers are free once its scores and V fragments have been
  // read, so the block synchronises there (not at the top of the next
  // iteration): that barrier also publishes tile it + 1's copy, and tile
  // it + 2's copy goes into the freed buffers right after it. The P V
  // products of tile it and the scores of tile it + 1 then follow each other
  // with no barrier between. `cur` walks the tiles being computed, `pre` the
  // tiles being copied, two ahead.
  Cur cur = at(si);
  if constexpr (FUSED) {
    while (cur.nt == 0 && cur.j + 1 < st.n) cur = at(cur.j + 1);
  }
  bool more = cur.nt > 0;
  Cur pre = cur;
  bool pre_more = more;
  if (more) {
    issue(pre, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    pre_more = advance(pre);
    if (pre_more) issue(pre, 1);
  }
  const int wrow_lo = q0 + w * 32, wrow_hi = wrow_lo + 31;
  const int wrow_last = min(wrow_hi, ql - 1);  // the wavefront's last row with a query
  for (int it = 0; more; ++it) {
    const int buf = it & 1;
    const int k0 = cur.kt * BN;
    const bool rows_any = wrow_lo < ql && wrow_last >= cur.rlo && wrow_lo < cur.rhi;
    const bool rows_all = wrow_lo >= cur.rlo && wrow_last < cur.rhi;
    const bool active = rows_any && !(cur.causal && k0 > wrow_hi);
    const bool need_mask = (k0 + BN > cur.kl) || (cur.causal && k0 + BN - 1 > wrow_lo) || !rows_all;
    bf16x8_t pb[KK2], vf[KK2][NMD];
    if (active) key_tile(cur, buf, need_mask, pb, vf);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (pre_more) {
      pre_more = advance(pre);
      if (pre_more) issue(pre, buf);
    }
    if (active) pv_tile(pb, vf);
    more = advance(cur);
  }

  const float lt = sum_halves(l_run);
  if constexpr (FUSED) {
    // every step is in: the bf16 output (through LDS, whole-row stores; the
    // K tiles are free) and the final LSE
    constexpr int SP = D * 2 + 16;
    // rows [0, FWD_BM / 2) stage in the K tiles, the rest in the V tiles
    constexpr int HALF = FWD_BM / 2;
    static_assert(HALF * SP <= (int)sizeof(Ks) && HALF * SP <= (int)sizeof(Vs), "output staging fits the tiles");
    auto srow = [&](int r) {
      return r < HALF ? reinterpret_cast<char*>(&Ks[0][0]) + r * SP : reinterpret_cast<char*>(&Vs[0][0]) + (r - HALF) * SP;
    };
    __syncthreads();  // every wavefront is done with the K and V tiles
    stage_row_bf16<D>(srow(w * 32 + l32), g, o, lt > 0.f ? 1.f / lt : 0.f);
    if (qrow < ql && g == 0)
      p.lse_out[(long long)head * p.ld_lse_out + qs + qrow] = lt > 0.f ? m_run * p.scale + __logf(lt) : NEG_INF_F;
    __syncthreads();
    uint16_t* const dst = p.out + (long long)(qs + q0) * p.ld_o + head * D;
    constexpr int UPR = D * 2 / 16;
    for (int u = tid; u < nq * UPR; u += BLOCK_THREADS) {
      const int r = u / UPR, cc = u - r * UPR;
      *reinterpret_cast<uint4*>(dst + (long long)r * p.ld_o + cc * 8) = *reinterpret_cast<const uint4*>(srow(r) + cc * 16);
    }
    return;
  }
  if (qrow < ql) step_epilogue<D>(p, st.o[si], st.lse[si], qs + qrow, head, g, o, m_run, lt);
}

// Padding rows of the final output: out 0, LSE -inf (every valid row is
// written by the last ring step's epilogue, or by the fused launch).
__global__ void __launch_bounds__(256) pad_rows_kernel(const int32_t* __restrict__ rowflags, uint16_t* __restrict__ out,
                                                       float* __restrict__ lse_out, int t_local, int hq, int d,
                                                       long long ld_lse_out) {
  const long long u_per_row = (long long)hq * d / 8;  // 16-byte units
  const long long n = (long long)t_local * u_per_row;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n; e += (long long)gridDim.x * blockDim.x) {
    const int t = (int)(e / u_per_row);
    if (rowflags[t] & RF_VALID) continue;
    const int u = (int)(e - (long long)t * u_per_row);
    reinterpret_cast<uint4*>(out + (long long)t * hq * d)[u] = make_uint4(0, 0, 0, 0);
    if (u < hq) lse_out[(long long)u * ld_lse_out + t] = NEG_INF_F;
  }
}

// Whether the forward runs every ring step in one fused launch (each block
// through all steps, merged in registers): when the steps' own launches
// would be short.
// Key rows per tile of the fused launch: 32-key tiles take 168 VGPRs and
// 41 KB of LDS, so three blocks share a CU (two with 64-key tiles); short
// shares are latency-bound and gain from the third (1.7-2.1% per step on
// the 16K packs), long ones lose (the per-tile costs double), so the
// per-step launches keep 64.
constexpr int FWD_BN_FUSED = 32;

static bool fwd_fused(const cp_attn_meta* m, int hq) {
  if (m->cp < 2) return false;
  long long mx = 0;
  for (int i = 0; i < m->cp; ++i) mx = std::max<long long>(mx, m->sum.tiles_fwd[i] * hq);
  return short_launches(mx, m->device);
}

// One launch of the ring steps listed in `st` (their blocks one after
// another; st.off is filled here from the steps' work-item counts), or
// (fused) one launch over the work items of entry 0, every block running
// through all the entries.
static cp_attn_status launch_fwd_steps(const cp_attn_meta* m, const FwdParams& p, FwdSteps st, int d, bool fused,
                                       hipStream_t strm) {
  long long blocks = 0;
  for (int j = 0; j < st.n; ++j) {
    st.off[j] = (int)blocks;
    if (!fused || j == 0) blocks += m->sum.tiles_fwd[st.step[j]] * p.hq;
    if (blocks > 0x7fffffffLL) return fail(CP_ATTN_ERR_UNSUPPORTED, "too many work items");
  }
  if (fused)
    for (int j = 0; j <= st.n; ++j) st.off[j] = 0;
  else
    st.off[st.n] = (int)blocks;
  if (blocks == 0) return CP_ATTN_OK;
  const dim3 grid((unsigned)blocks), blk(BLOCK_THREADS);
  timing_begin(strm, fused ? "fwd_fused" : "fwd_step");
  if (d == 128) {
    if (fused)
      hipLaunchKernelGGL((fwd_step_kernel<128, true, FWD_BN_FUSED>), grid, blk, 0, strm, p, st);
    else
      hipLaunchKernelGGL((fwd_step_kernel<128, false, 64>), grid, blk, 0, strm, p, st);
  } else {
    if (fused)
      hipLaunchKernelGGL((fwd_step_kernel<64, true, FWD_BN_FUSED>), grid, blk, 0, strm, p, st);
    else
      hipLaunchKernelGGL((fwd_step_kernel<64, false, 64>), grid, blk, 0, strm, p, st);
  }
  timing_end(strm);
  return hip_check(hipGetLastError(), "fwd_step launch");
}

// Ring step i's entry of a FwdSteps list.
static void add_step(const cp_attn_meta* m, FwdSteps& st, int i, const void* const* k_shards,
                     const void* const* v_shards, float* o, float* lse) {
  const int j = st.n++;
  const int s = m->sum.step_src[i];
  st.k[j] = (const uint16_t*)k_shards[s];
  st.v[j] = (const uint16_t*)v_shards[s];
  st.items[j] = m->d_tab + m->lay.fwd_tiles + (int64_t)i * m->lay.fwd_cap * 2;
  st.o[j] = o;
  st.lse[j] = lse;
  st.step[j] = i;
  st.kind[j] = m->sum.step_kind[i];
}

static unsigned stream_blocks(long long n, int per_block) {
  long long b = (n + per_block - 1) / per_block;
  if (b < 1) b = 1;
  return (unsigned)std::min<long long>(b, 8192);
}

}  // namespace cpattn

using namespace cpattn;

extern "C" size_t cp_attn_workspace_bytes(const cp_attn_meta* m, int32_t hq, int32_t hkv, int32_t d, int32_t pass) {
  (void)hkv;
  if (!m || hq <= 0 || d <= 0) return 0;
  const size_t tl = (size_t)m->sum.t_local;
  const size_t o = tl * hq * d * sizeof(float);
  const size_t l = ((tl * hq * sizeof(float)) + 255) & ~size_t(255);
  const size_t o_al = (o + 255) & ~size_t(255);
  if (pass == 0)  // the running accumulator (out, lse); the fused launch of short shares leaves it untouched
    return o_al + l;
  return 2 * l;                            // per-row lse and -D = -rowsum(dO * O)
}

static cp_attn_status check_common(const cp_attn_meta* m, const void* q, const void* const* ks, const void* const* vs,
                                   int hq, int hkv, int d, int causal) {
  if (!m) return fail(CP_ATTN_ERR_INVALID_ARG, "meta is NULL");
  if (!q || !ks || !vs) return fail(CP_ATTN_ERR_INVALID_ARG, "NULL tensor argument");
  if (causal != 1) return fail(CP_ATTN_ERR_UNSUPPORTED, "only causal attention is supported");
  if (d != 64 && d != 128) return fail(CP_ATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return fail(CP_ATTN_ERR_INVALID_ARG, "hq must be a positive multiple of hkv");
  for (int s = 0; s < m->cp; ++s)
    if (!ks[s] || !vs[s]) return fail(CP_ATTN_ERR_INVALID_ARG, "NULL K/V shard pointer");
  if (((uintptr_t)q) & 15) return fail(CP_ATTN_ERR_INVALID_ARG, "q must be 16-byte aligned");
  for (int s = 0; s < m->cp; ++s)
    if ((((uintptr_t)ks[s]) | ((uintptr_t)vs[s])) & 15) return fail(CP_ATTN_ERR_INVALID_ARG, "K/V shards must be 16-byte aligned");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != m->device)
    return fail(CP_ATTN_ERR_INVALID_ARG, "current device differs from the metadata's device");
  return CP_ATTN_OK;
}

extern "C" cp_attn_status cp_attn_fwd(const cp_attn_meta* m, const void* q, const void* const* k_shards,
                                      const void* const* v_shards, int32_t hq, int32_t hkv, int32_t d,
                                      float softmax_scale, int32_t causal, void* out, float* lse, void* workspace,
                                      size_t ws_bytes, void* stream) {
  set_error("");
  cp_attn_status rc = check_common(m, q, k_shards, v_shards, hq, hkv, d, causal);
  if (rc != CP_ATTN_OK) return rc;
  if (!out || !lse) return fail(CP_ATTN_ERR_INVALID_ARG, "NULL output");
  if (!(softmax_scale > 0.f) || !(softmax_scale < 1e30f)) return fail(CP_ATTN_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
  if (((uintptr_t)out) & 15) return fail(CP_ATTN_ERR_INVALID_ARG, "out must be 16-byte aligned");
  const size_t need = cp_attn_workspace_bytes(m, hq, hkv, d, 0);
  if (!workspace || ws_bytes < need) return fail(CP_ATTN_ERR_WORKSPACE, "forward workspace missing or too small");
  if (((uintptr_t)workspace) & 255) return fail(CP_ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const int tl = m->sum.t_local;
  if (tl == 0) return CP_ATTN_OK;
  if ((long long)hq * d * 2 > (1ll << 20))
    return fail(CP_ATTN_ERR_UNSUPPORTED, "a row of all heads must stay within 1 MiB");
  hipStream_t st_ = (hipStream_t)stream;
  const size_t o_al = (((size_t)tl * hq * d * sizeof(float)) + 255) & ~size_t(255);
  char* ws = (char*)workspace;
  const int32_t* rowflags = m->d_tab + m->lay.rowflags;

  FwdParams base{};
  base.q = (const uint16_t*)q;
  base.steps = m->d_tab + m->lay.steps;
  base.B = m->B;
  base.hq = hq;
  base.group = hq / hkv;
  base.ld_q = (long long)hq * d;
  base.ld_kv = (long long)hkv * d;
  base.scale = softmax_scale;
  base.c_log2 = softmax_scale * LOG2E_F;
  base.ld_o = (long long)hq * d;
  base.ld_lse = tl;
  base.rowflags = rowflags;
  base.out = (uint16_t*)out;
  base.lse_out = lse;
  base.ld_lse_out = (long long)m->t_alloc;
  if (fwd_fused(m, hq)) {
    // every step in one launch, the causal step first (its work items are
    // the blocks' rows), then the others in ring order
    FwdSteps st{};
    for (int i = 0; i < m->cp; ++i) add_step(m, st, i, k_shards, v_shards, nullptr, nullptr);
    FwdParams p = base;
    p.mode = 2;
    if ((rc = launch_fwd_steps(m, p, st, d, true, st_)) != CP_ATTN_OK) return rc;
  } else {
    // In order: each step folds its partial into the accumulator in its own
    // epilogue. The steps are independent on one device, so the second-chunk
    // steps (kind 2) run first, then the kind-1 steps, and the causal step,
    // which covers every valid row of both chunks, runs last and writes the
    // bf16 output and the final LSE.
    int order[CP_ATTN_MAX_CP], n_order = 0;
    for (int want : {2, 1, 0})
      for (int i = 0; i < m->cp; ++i)
        if (m->sum.step_kind[i] == want) order[n_order++] = i;
    bool acc_first = false, acc_second = false;
    for (int k = 0; k < n_order; ++k) {
      const int i = order[k];
      const int kind = m->sum.step_kind[i];
      FwdParams p = base;
      p.mode = (k == n_order - 1) ? 2 : 1;
      p.acc_first = acc_first;
      p.acc_second = acc_second;
      FwdSteps one{};
      add_step(m, one, i, k_shards, v_shards, (float*)ws, (float*)(ws + o_al));
      if ((rc = launch_fwd_steps(m, p, one, d, false, st_)) != CP_ATTN_OK) return rc;
      acc_second = true;
      if (kind != 2) acc_first = true;
    }
  }
  if (m->sum.valid_rows < tl) {
    timing_begin(st_, "pad_rows");
    hipLaunchKernelGGL(pad_rows_kernel, dim3(stream_blocks((long long)tl * hq * d / 8, 256)), dim3(256), 0, st_,
                       rowflags, (uint16_t*)out, lse, tl, hq, d, (long long)m->t_alloc);
    timing_end(st_);
    rc = hip_check(hipGetLastError(), "pad_rows launch");
  }
  return rc;
}
