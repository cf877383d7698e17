// Backward of one CP rank's share on MFMA.
//
// Per ring step (the same step tables as the forward): a dK/dV kernel whose
// blocks own 128 key rows of the source shard and loop over the step's query
// rows (and over the query heads of a GQA group), and a dQ kernel whose blocks
// own 128 query rows and loop over the step's key rows. Both recompute the
// probabilities from the forward's final LSE, P = exp(scale q.k - lse), and
// use dS = P (dP - D) with D = rowsum(dO * out). THD gradient tail zeroing
// ("[PyTorch][Attention] THD P2P context-parallel regression ...", sections
// "Describe the bug" and "Expected behavior") is one extra launch made only
// when the metadata reports rows past the valid end (t_alloc > T_local).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "internal.h"
#include "kern_common.h"

namespace cpattn {

// What both backward kernels share; the per-step shards and outputs come in
// DkdvSteps / DqSteps.
struct BwdParams {
  const uint16_t* q;
  const uint16_t* dout;
  const float* lse2;  // forward LSE in exp2 units, fp32 [hq, ld_ldv] (+inf on padding rows)
  const float* negd;  // -D = -rowsum(dO * out), fp32 [hq, ld_ldv] (0 on padding rows)
  long long ld_ldv;
  const int32_t* steps;  // every step's sequence tables: [step][q_start, q_len, kv_start, kv_len][B]
  int B;
  const int32_t* slot;   // cu_seqlens_padded / CP (slot starts, B + 1)
  const int32_t* items;  // dQ work items: (sequence, 128-row tile) of the causal step's rows
  int hq, hkv, group;
  long long ld_q, ld_kv;
  float scale, c_log2;
  uint16_t* dq;          // bf16 [t_alloc, hq, D]
};

// Per (head, local row): the forward's LSE in exp2 units and
// -D = -rowsum(dO * out), as two fp32 planes [hq, t_local]; padding rows get
// (+inf, 0), so their probabilities vanish. 16 lanes cover one (row, head)
// of D = 128 (8 lanes for D = 64).
__global__ void __launch_bounds__(256) bwd_pre_kernel(const uint16_t* __restrict__ dout, const uint16_t* __restrict__ out,
                                                      const float* __restrict__ lse, long long ld_lse,
                                                      const int32_t* __restrict__ rowflags, float* __restrict__ lse2,
                                                      float* __restrict__ negd, int t_local, int hq, int d) {
  const int lanes = d / 8;
  const long long n = (long long)t_local * hq * lanes;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n; e += (long long)gridDim.x * blockDim.x) {
    const long long rh = e / lanes;
    const int part = (int)(e - rh * lanes);
    const int t = (int)(rh / hq);
    const int h = (int)(rh - (long long)t * hq);
    const bool valid = rowflags[t] & RF_VALID;
    float acc = 0.f;
    if (valid) {
      const uint4 a = *reinterpret_cast<const uint4*>(dout + rh * d + part * 8);
      const uint4 b = *reinterpret_cast<const uint4*>(out + rh * d + part * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = u4_get(a, w), y = u4_get(b, w);
        acc += __uint_as_float(x << 16) * __uint_as_float(y << 16);
        acc += __uint_as_float(x & 0xffff0000u) * __uint_as_float(y & 0xffff0000u);
      }
    }
    for (int off = lanes >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (part == 0) {
      const long long i = (long long)h * t_local + t;
      lse2[i] = valid ? lse[(long long)h * ld_lse + t] * LOG2E_F : __builtin_huge_valf();
      negd[i] = -acc;
    }
  }
}

// The ring steps' K / V shards for the dQ kernel: step i reads shard
// k[i] / v[i] through step i's sequence tables.
struct DqSteps {
  const uint16_t* k[CP_ATTN_MAX_CP];
  const uint16_t* v[CP_ATTN_MAX_CP];
  int kind[CP_ATTN_MAX_CP];
  int n;
};

// dQ of every ring step at once: dQ = scale sum_i dS_i K_i summed over the
// steps in registers, written once in bf16. Block = NWAVES wavefronts x 32
// query rows of one head (a 128-row tile of the rows the causal step covers,
// which are all the valid rows of the sequence's slot). The block walks the
// steps' key ranges in one pipeline of 64-key tiles: K and V are copied
// straight into padded LDS tiles (double-buffered, the next tile's copy may
// belong to the next step). Row-major reads of K and V feed the transposed
// scores S^T = K Q^T and dP^T = V dO^T (lane = one query row); transposing
// reads of the same K tile feed dQ^T = K^T dS^T. A step that covers only the
// second chunk's rows (s > rank) leaves the other rows out through their
// LSE (+inf: their probabilities vanish). Keys past a step's key range read
// as zeros, so their K^T rows contribute nothing and need no mask.
template <int D>
__global__ void __launch_bounds__(BLOCK_THREADS, 8 / NWAVES) bwd_dq_kernel(BwdParams p, DqSteps st) {
  constexpr int BM = FWD_BM, BN = 64;
  constexpr int NKK = D / 16, NMD = D / 32;
  using KCopy = TileCopy<D, false, BN, NWAVES, true>;  // K read both ways: permuted rows (V too, same plan)
  // one LDS array per buffer (its K tile, then its V tile), always named
  // statically, so the compiler sees that this tile's reads cannot touch the
  // buffer whose copy is in flight
  __shared__ __attribute__((aligned(1024))) uint16_t T0[KCopy::BYTES];
  __shared__ __attribute__((aligned(1024))) uint16_t T1[KCopy::BYTES];
  auto ks_of = [&](auto b) { return decltype(b)::value ? T1 : T0; };
  auto vs_of = [&](auto b) { return (decltype(b)::value ? T1 : T0) + KCopy::BYTES / 2; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index (uniform)
  int item, head;
  map_block(blockIdx.x, p.hq, item, head);
  const int sb = p.items[2 * item], tile = p.items[2 * item + 1];
  const int B = p.B;
  // step tables: [step][q_start, q_len, kv_start, kv_len][sequence], read
  // once into LDS: moving on to the next step mid-loop then reads LDS and
  // does not wait for the tile copies in flight (a global read would: the
  // load counter retires in order)
  __shared__ int step_tab[4 * CP_ATTN_MAX_CP];
  for (int i = 0; i < st.n; ++i)
    if (tid < 4) step_tab[4 * i + tid] = p.steps[(long long)i * 4 * B + tid * B + sb];
  __syncthreads();
  auto tab = [&](int i, int f) { return step_tab[4 * i + f]; };
  const int base = tab(0, 0), ql0 = tab(0, 1);  // the causal step covers every valid row of the slot
  const int q0 = tile * BM;
  const int nq = min(BM, ql0 - q0);
  const int kvh = head / p.group;
  const float c = p.c_log2;

  const int qrow = q0 + w * 32 + l32;  // relative to the slot
  const bool qok = qrow < ql0;
  bf16x8_t qf[NKK], df[NKK];
  {
    const long long roff = (long long)(base + (qok ? qrow : 0)) * p.ld_q + head * D + g * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[kk] = as_bf16x8(qok ? *reinterpret_cast<const uint4*>(p.q + roff + kk * 16) : make_uint4(0, 0, 0, 0));
      df[kk] = as_bf16x8(qok ? *reinterpret_cast<const uint4*>(p.dout + roff + kk * 16) : make_uint4(0, 0, 0, 0));
    }
  }
  const long long li = (long long)head * p.ld_ldv + base + qrow;
  const float lse2_row = qok ? p.lse2[li] : __builtin_huge_valf();
  const float dq_d = qok ? -p.negd[li] : 0.f;

  f32x16_t acc[NMD];
#pragma unroll
  for (int md = 0; md < NMD; ++md) acc[md] = zero16();
  // -D of the lane's row: every dP^T chain starts from it (the first MFMA
  // reads it as its accumulator input, so dP^T - D costs no VALU)
  f32x16_t negd16;
#pragma unroll
  for (int j = 0; j < 16; ++j) negd16[j] = -dq_d;

  const int ldb = (int)(p.ld_kv * 2);
  KCopy kc;
  kc.init(ldb, w, lane);
  // a step's view for this block: its rows (slot-relative [rlo, rhi)), its
  // keys, how many 64-key tiles the block visits (0: the step does not
  // reach the block's rows), where its K and V rows start and the byte end
  // of its key range (end32; -1 when a tile offset could pass 2^31, which
  // then takes 64-bit arithmetic)
  struct View {
    int rlo, rhi, kl, nt, causal, end32;
    const uint16_t* kb;
    const uint16_t* vb;
  };
  auto view = [&](int i) {
    View v;
    v.rlo = tab(i, 0) - base;
    v.rhi = v.rlo + tab(i, 1);
    v.kl = tab(i, 3);
    v.causal = st.kind[i] == 0;
    const int lo = max(q0, v.rlo), hi = min(q0 + nq, v.rhi);
    const int n_keys = hi <= lo ? 0 : (v.causal ? min(v.kl, q0 + nq) : v.kl);
    v.nt = (n_keys + BN - 1) / BN;
    const long long kvs = tab(i, 2);
    v.kb = st.k[i] + kvs * p.ld_kv + kvh * D;
    v.vb = st.v[i] + kvs * p.ld_kv + kvh * D;
    const long long end = (long long)v.kl * ldb;
    v.end32 = end <= 0x7fffffffLL ? (int)end : -1;
    return v;
  };
  auto issue = [&](const View& v, int kt, auto buf) {
    if (v.end32 >= 0) {
      const int off = kt * (BN * ldb);  // below end32, so below 2^31
      kc.copy(rsrc_from32(v.kb, off, v.end32), ks_of(buf), w);
      kc.copy(rsrc_from32(v.vb, off, v.end32), vs_of(buf), w);
    } else {
      const long long off = (long long)kt * BN * ldb, end = (long long)v.kl * ldb;
      kc.copy(rsrc_from(v.kb, off, end), ks_of(buf), w);
      kc.copy(rsrc_from(v.vb, off, end), vs_of(buf), w);
    }
  };
  // the first step with work, then (step, tile) in order
  int i = 0;
  View cur = view(0);
  while (cur.nt == 0 && i + 1 < st.n) cur = view(++i);
  if (cur.nt > 0) issue(cur, 0, Buf<0>{});
  const int wrow_lo = q0 + w * 32, wrow_hi = wrow_lo + 31;
  int kt = 0;
  // one tile in buffer `buf` (the loop below alternates the buffers); every
  // next tile's copy goes to the other buffer, which the next tile's barrier
  // publishes
  auto tile_step = [&](auto buf) {
    // the tile after this one, possibly the next step's first
    int ni = i, nkt = kt + 1;
    View nxt = cur;
    if (nkt >= cur.nt) {
      nkt = 0;
      nxt.nt = 0;
      while (nxt.nt == 0 && ni + 1 < st.n) nxt = view(++ni);
    }
    const bool more = nxt.nt > 0;
    const Buf<1 - decltype(buf)::value> other{};
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int k0 = kt * BN;
    const bool active = !(cur.causal && k0 > wrow_hi) && wrow_lo < min(ql0, cur.rhi) && wrow_hi >= cur.rlo;
    // the next tile's copy is issued after this tile's score products (the
    // address arithmetic then fills the wait for their results); idle
    // wavefronts issue their share at once
    if (!active && more) issue(nxt, nkt, other);
    if (active) {
      // rows outside this step's query range take no part in it
      const float lse2 = (qrow >= cur.rlo && qrow < cur.rhi) ? lse2_row : __builtin_huge_valf();
      f32x16_t s[2], dp[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = zero16();
        dp[mb] = negd16;
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          s[mb] = mfma32x32x16(lds_read_row<D, true>(ks_of(buf), mb * 32 + l32, 2 * kk + g), qf[kk], s[mb]);
      }
      if (more) issue(nxt, nkt, other);
      if (cur.causal && k0 + BN - 1 > wrow_lo) {
        // keys after the lane's row (a real branch, kept out of
        // if-conversion; only the tiles on a wavefront's diagonal take it)
        __asm__ volatile("" ::: "memory");
        const int rel = qrow - k0 - 4 * g;  // element (mb, j): key offset 32 mb + 8 (j / 4) + j % 4
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j) s[mb][j] = (mb * 32 + (j >> 2) * 8 + (j & 3) <= rel) ? s[mb][j] : NEG_INF_F;
      }
      // dP^T products with the probabilities computed beside them (4 per k
      // step): the exponentials issue while the matrix unit works, instead
      // of after both chains
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          dp[mb] = mfma32x32x16(lds_read_row<D, true>(vs_of(buf), mb * 32 + l32, 2 * kk + g), df[kk], dp[mb]);
#pragma unroll
        for (int e = 0; e < 32 / NKK; ++e) {
          const int j = kk * (32 / NKK) + e;
          s[j >> 4][j & 15] = fast_exp2(fmaf(s[j >> 4][j & 15], c, -lse2));
        }
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[mb][j] *= dp[mb][j];  // dS^T = P (dP - D)
#pragma unroll
      for (int kk2 = 0; kk2 < BN / 16; ++kk2) {
        const bf16x8_t ds = pack8_bf16(s[kk2 >> 1], 8 * (kk2 & 1));
#pragma unroll
        for (int md = 0; md < NMD; ++md)
          acc[md] = mfma32x32x16(lds_read_tr<D, false, true, true>(ks_of(buf), kk2 * 16, md * 32, lane), ds, acc[md]);
      }
    }
    i = ni;
    kt = nkt;
    cur = nxt;
  };
  while (cur.nt > 0) {
    tile_step(Buf<0>{});
    if (cur.nt == 0) break;
    tile_step(Buf<1>{});
  }
  // bf16 dQ through LDS (the K tiles are free), whole-row stores
  constexpr int SP = D * 2 + 16;
  static_assert(BM * SP <= (int)sizeof(T0), "dQ staging fits one buffer");
  char* const stage = reinterpret_cast<char*>(&T0[0]);
  __syncthreads();  // every wavefront is done with the K and V tiles
  stage_row_bf16<D>(stage + (w * 32 + l32) * SP, g, acc, p.scale);
  __syncthreads();
  store_rows<D, SP, BLOCK_THREADS>(stage, nq, p.dq + (long long)(base + q0) * p.hq * D + head * D, (long long)p.hq * D, tid);
}

// dK/dV of one ring step for the source shard's key rows. Block = NWAVES
// wavefronts x DKDV_KB blocks of 32 key rows of one KV head (DKDV_BN keys),
// K in registers and V in LDS; loops over the query heads of the group and
// the step's query rows in tiles of 32. Q and dO tiles are copied straight
// into padded LDS tiles (double-buffered) together with the rows' LSE and -D.
// Row-major reads feed S = Q K^T and dP = dO V^T (lane = one key column);
// transposing reads feed dV^T += dO^T P and dK^T += Q^T dS (lane = one key row
// of the output). Each Q / dO fragment read from LDS serves all of a
// wavefront's key blocks. Query rows past the step's range read as zeros
// (Q = dO = D = 0), which makes their dS and P.dO contributions vanish; key
// rows past the key range are computed but written as zeros. Rows of the part
// outside the step's key range are written as zeros too, so the whole
// shard-s part is defined.
// The ring steps' shards and outputs for the dK/dV kernel: blocks
// [off[i], off[i + 1]) work on step i (K / V shard k[i] / v[i], its part
// dk[i] / dv[i], work items items[i]).
struct DkdvSteps {
  const uint16_t* k[CP_ATTN_MAX_CP];
  const uint16_t* v[CP_ATTN_MAX_CP];
  uint16_t* dk[CP_ATTN_MAX_CP];
  uint16_t* dv[CP_ATTN_MAX_CP];
  const int32_t* items[CP_ATTN_MAX_CP];
  int step[CP_ATTN_MAX_CP];  // ring step index (its sequence tables)
  int kind[CP_ATTN_MAX_CP];
  int off[CP_ATTN_MAX_CP + 1];
  int n;
};

template <int D, bool BIG>
__global__ void __launch_bounds__(BLOCK_THREADS, (8 / NWAVES / DKDV_KB) > 0 ? 8 / NWAVES / DKDV_KB : 1)
    bwd_dkdv_kernel(BwdParams p, DkdvSteps sts) {
  constexpr int KB = DKDV_KB;
  constexpr int BK = DKDV_BN, BQ = 32;
  constexpr int NKK = D / 16, NMD = D / 32;
  // Q and dO are read both ways: permuted rows. The first half of the
  // wavefronts copies the Q tile and the second half the dO tile (whole
  // chunk counts per wavefront, no per-chunk guards)
  static_assert(NWAVES % 2 == 0, "the Q and dO tiles are copied by half the wavefronts each");
  using QCopy = TileCopy<D, false, BQ, NWAVES / 2, true>;
  using VCopy = TileCopy<D, false, BK, NWAVES>;
  __shared__ __attribute__((aligned(1024))) uint16_t Qs[2][QCopy::BYTES / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t Ds[2][QCopy::BYTES / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t Vt[VCopy::BYTES / 2];  // the block's V rows
  __shared__ __attribute__((aligned(16))) float LD[2][2 * BQ];  // per buffer: the rows' lse * log2(e), then -D

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index (uniform)
  // this block's ring step (every block of one step shares it)
  int si = 0;
  while (si + 1 < sts.n && (int)blockIdx.x >= sts.off[si + 1]) ++si;
  si = __builtin_amdgcn_readfirstlane(si);
  const int32_t* tabs = p.steps + (long long)sts.step[si] * 4 * p.B;
  const bool causal = sts.kind[si] == 0;
  int item, kvh;
  map_block((int)blockIdx.x - sts.off[si], p.hkv, item, kvh);
  const int sb = sts.items[si][2 * item], tile = sts.items[si][2 * item + 1];
  const int qs = tabs[sb], ql = tabs[p.B + sb], kvs = tabs[2 * p.B + sb], kl = tabs[3 * p.B + sb];
  const int slot_len = p.slot[sb + 1] - p.slot[sb];
  const int k0 = tile * BK;
  const int rows_here = min(BK, slot_len - k0);
  const int nk = max(0, min(BK, kl - k0));
  const int wr0 = w * 32 * KB;  // the wavefront's first key row within the block
  const float c = p.c_log2;

  f32x16_t dk[KB][NMD], dv[KB][NMD];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int md = 0; md < NMD; ++md) {
      dk[kb][md] = zero16();
      dv[kb][md] = zero16();
    }

  // query tiles to visit: causal steps skip tiles entirely before this key tile
  const int qt_begin = (causal && nk > 0) ? (k0 / BQ) : 0;
  const int qt_end = nk > 0 ? (ql + BQ - 1) / BQ : 0;
  const int n_qt = max(0, qt_end - qt_begin);
  const int n_iter = n_qt * p.group;

  if (n_iter > 0) {
    // K rows of this lane's keys in registers, the block's V rows in LDS
    // (every lane loads from a valid row, row 0 of the range for keys past
    // it, and zeroes those afterwards: the loads issue back to back, with no
    // branch between them)
    bf16x8_t kf[KB][NKK];
    const uint16_t* const kshard = sts.k[si];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = k0 + wr0 + kb * 32 + l32;
      const bool ok = key < kl;
      const uint4* const src =
          reinterpret_cast<const uint4*>(kshard + (long long)(kvs + (ok ? key : 0)) * p.ld_kv + kvh * D + g * 8);
      uint4 u[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) u[kk] = src[2 * kk];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) kf[kb][kk] = as_bf16x8(ok ? u[kk] : make_uint4(0, 0, 0, 0));
    }
    {
      const int ldkv = (int)(p.ld_kv * 2);
      VCopy vcp;
      vcp.init(ldkv, w, lane);
      vcp.copy(rsrc_from(sts.v[si] + (long long)(kvs + k0) * p.ld_kv + kvh * D, 0, (long long)nk * ldkv), Vt, w);
    }
    const int ldb = (int)(p.ld_q * 2);
    const long long q_end = (long long)ql * ldb, ld_end = (long long)ql * 4;
    QCopy qc;  // the same plan serves Q and dO
    const int cw = w % (NWAVES / 2);  // the wavefront's index among the tile's copiers
    qc.init(ldb, cw, lane);
    // the step's first query row, and the head-to-head strides in bytes
    const char* q_base = reinterpret_cast<const char*>(p.q + (long long)qs * p.ld_q);
    const char* do_base = reinterpret_cast<const char*>(p.dout + (long long)qs * p.ld_q);
    const char* l_base = reinterpret_cast<const char*>(p.lse2 + qs);
    const char* n_base = reinterpret_cast<const char*>(p.negd + qs);
    const long long ld_head = p.ld_ldv * 4;
    // query head hh, query tile qt: Q and dO rows, and the rows' lse and -D
    // (128 bytes each, copied by 16 lanes of wavefront 0)
    // BIG: local query tensors of 2 GiB or more need 64-bit offsets; below
    // that the cheaper 32-bit scalar arithmetic serves
    auto issue = [&](int hh, int qt, int buf) {
      const bool first = w < NWAVES / 2;  // uniform: Q tile, else dO tile
      const char* base = (first ? q_base : do_base) + hh * (D * 2);
      uint16_t* dst = first ? Qs[buf] : Ds[buf];
      if constexpr (BIG)
        qc.copy(rsrc_from(base, (long long)qt * (BQ * ldb), q_end), dst, cw);
      else
        qc.copy(rsrc_from32(base, qt * (BQ * ldb), (int)q_end), dst, cw);
      if (w == 0) {
        const int toff = qt * (BQ * 4);
        const __amdgpu_buffer_rsrc_t lr = rsrc_from32(l_base + hh * ld_head, toff, (int)ld_end);
        const __amdgpu_buffer_rsrc_t dr = rsrc_from32(n_base + hh * ld_head, toff, (int)ld_end);
        if (lane < BQ / 4)
          load_lds16(lr, &LD[buf][0], lane * 16);
        else if (lane < BQ / 2)
          load_lds16(dr, &LD[buf][0], (lane - BQ / 4) * 16);
      }
    };
    static_assert(sizeof(LD[0]) == BQ * 8, "lse / -D tile layout");

    // query tiles last to first, and for each tile the group's query heads in
    // turn: every key block of a KV head starts on the same tile and the
    // blocks move down the query rows together, also at the causal step,
    // where their sweeps end at different tiles (shared Q / dO tiles in L2)
    const int h_first = kvh * p.group, h_last = h_first + p.group - 1;
    int hh = h_first, qt = qt_end - 1;
    issue(hh, qt, 0);
    const int wkey_hi = k0 + wr0 + 32 * KB - 1;
    for (int it = 0; it < n_iter; ++it) {
      const int buf = it & 1;
      const int cur_qt = qt;
      if (hh == h_last) {
        hh = h_first;
        --qt;
      } else {
        ++hh;
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (it + 1 < n_iter) issue(hh, qt, buf ^ 1);
      // every wavefront computes every tile (no branch around the MFMAs, so
      // the accumulators stay in place across iterations); tiles wholly in
      // the future of a wavefront's keys are zeroed by the causal mask
      const int qlo = cur_qt * BQ;
      {
        // S = Q K^T and dP - D = dO V^T - D: rows q (this lane: 16 of them),
        // column key; the dP accumulators start at -D of their rows
        f32x16_t s[KB], dp[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          s[kb] = zero16();
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const float4 nd = *reinterpret_cast<const float4*>(&LD[buf][BQ + jq * 8 + g * 4]);
            dp[kb][4 * jq + 0] = nd.x;
            dp[kb][4 * jq + 1] = nd.y;
            dp[kb][4 * jq + 2] = nd.z;
            dp[kb][4 * jq + 3] = nd.w;
          }
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const bf16x8_t qa = lds_read_row<D, true>(Qs[buf], l32, 2 * kk + g);
          const bf16x8_t da = lds_read_row<D, true>(Ds[buf], l32, 2 * kk + g);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            s[kb] = mfma32x32x16(qa, kf[kb][kk], s[kb]);
            dp[kb] = mfma32x32x16(da, lds_read_row<D>(Vt, wr0 + kb * 32 + l32, 2 * kk + g), dp[kb]);
          }
        }
        // the first query slice's transposed fragments are read now, so
        // their LDS latency hides behind the softmax (the scheduling fence
        // keeps the compiler from sinking the reads again)
        bf16x8_t ta0[NMD], tq0[NMD];
#pragma unroll
        for (int md = 0; md < NMD; ++md) {
          ta0[md] = lds_read_tr<D, false, true>(Ds[buf], 0, md * 32, lane);
          tq0[md] = lds_read_tr<D, false, true>(Qs[buf], 0, md * 32, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (causal && qlo < wkey_hi) {
          // query rows before a lane's key (a real branch, kept out of
          // if-conversion; only a wavefront's first tiles take it)
          __asm__ volatile("" ::: "memory");
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            // element j: query row offset 8 (j / 4) + j % 4 from qlo + 4 g
            const int rel = k0 + wr0 + kb * 32 + l32 - qlo - 4 * g;
#pragma unroll
            for (int j = 0; j < 16; ++j) s[kb][j] = ((j >> 2) * 8 + (j & 3) >= rel) ? s[kb][j] : NEG_INF_F;
          }
        }
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          // rows 8 jq + 4 g + e, e = 0..3
          const float4 l4 = *reinterpret_cast<const float4*>(&LD[buf][jq * 8 + g * 4]);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = 4 * jq + e;
              const float pv = fast_exp2(fmaf(s[kb][j], c, -lv[e]));
              s[kb][j] = pv;               // P
              dp[kb][j] = pv * dp[kb][j];  // dS = P (dP - D), in place
            }
        }
        // dV^T += dO^T P, dK^T += Q^T dS (k = query rows, two slices of 16)
#pragma unroll
        for (int kq = 0; kq < BQ / 16; ++kq) {
          bf16x8_t pb[KB], db[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            pb[kb] = pack8_bf16(s[kb], 8 * kq);
            db[kb] = pack8_bf16(dp[kb], 8 * kq);
          }
#pragma unroll
          for (int md = 0; md < NMD; ++md) {
            const bf16x8_t ta = kq == 0 ? ta0[md] : lds_read_tr<D, false, true>(Ds[buf], kq * 16, md * 32, lane);
            const bf16x8_t tq = kq == 0 ? tq0[md] : lds_read_tr<D, false, true>(Qs[buf], kq * 16, md * 32, lane);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              dv[kb][md] = mfma32x32x16(ta, pb[kb], dv[kb][md]);
              dk[kb][md] = mfma32x32x16(tq, db[kb], dk[kb][md]);
            }
          }
        }
      }
    }
  }
  // The block's key rows leave through LDS (the Q, dO and V tiles are free
  // now): each lane parks its rows' dK / dV values (d = 32 md + 8 (j / 4) +
  // 4 g + (j % 4)) in padded row-major staging tiles, then every global
  // store writes 16 bytes of a whole row, 16 lanes per row of D = 128.
  constexpr int SP = D * 2 + 16;  // staging row pitch in bytes
  static_assert(BK * SP <= (int)sizeof(Vt), "dK staging fits the V tile");
  static_assert((BK / 2) * SP <= (int)sizeof(Qs) && (BK / 2) * SP <= (int)sizeof(Ds), "dV staging fits Q and dO");
  char* const stk = reinterpret_cast<char*>(Vt);
  auto stv = [&](int r) {
    return r < BK / 2 ? reinterpret_cast<char*>(&Qs[0][0]) + r * SP : reinterpret_cast<char*>(&Ds[0][0]) + (r - BK / 2) * SP;
  };
  __syncthreads();  // every wavefront is done with the Q, dO and V tiles
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int r = wr0 + kb * 32 + l32;
    const bool ok = k0 + r < kl;  // key rows past the step's key range are written as zeros
#pragma unroll
    for (int md = 0; md < NMD; ++md)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint2 a = make_uint2(0, 0), b = make_uint2(0, 0);
        if (ok) {
          a.x = pack2_bf16(dk[kb][md][4 * jj] * p.scale, dk[kb][md][4 * jj + 1] * p.scale);
          a.y = pack2_bf16(dk[kb][md][4 * jj + 2] * p.scale, dk[kb][md][4 * jj + 3] * p.scale);
          b.x = pack2_bf16(dv[kb][md][4 * jj], dv[kb][md][4 * jj + 1]);
          b.y = pack2_bf16(dv[kb][md][4 * jj + 2], dv[kb][md][4 * jj + 3]);
        }
        const int cb = (md * 32 + jj * 8 + g * 4) * 2;
        *reinterpret_cast<uint2*>(stk + r * SP + cb) = a;
        *reinterpret_cast<uint2*>(stv(r) + cb) = b;
      }
  }
  __syncthreads();
  constexpr int UPR = D * 2 / 16;  // 16-byte units per row
  for (int u = tid; u < rows_here * UPR; u += BLOCK_THREADS) {
    const int r = u / UPR, c = u - r * UPR;
    const long long e = (long long)(kvs + k0 + r) * p.ld_kv + kvh * D + c * 8;
    *reinterpret_cast<uint4*>(sts.dk[si] + e) = *reinterpret_cast<const uint4*>(stk + r * SP + c * 16);
    *reinterpret_cast<uint4*>(sts.dv[si] + e) = *reinterpret_cast<const uint4*>(stv(r) + c * 16);
  }
}

// dQ padding rows (no valid token; no dQ block covers them) set to 0;
// launched only when the share has such rows.
__global__ void __launch_bounds__(256) dq_pad_rows_kernel(const int32_t* __restrict__ rowflags,
                                                          uint16_t* __restrict__ dq, int t_local, int hq, int d) {
  const long long u_per_row = (long long)hq * d / 8;  // 16-byte units
  const long long n = (long long)t_local * u_per_row;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n; e += (long long)gridDim.x * blockDim.x) {
    const int t = (int)(e / u_per_row);
    if (rowflags[t] & RF_VALID) continue;
    reinterpret_cast<uint4*>(dq)[e] = make_uint4(0, 0, 0, 0);
  }
}

struct TailPtrs {
  uint16_t* p[1 + 2 * CP_ATTN_MAX_CP];
};

// Zero rows [t_local, t_alloc) of dQ and of every dK/dV part (16-byte stores).
__global__ void __launch_bounds__(256) tail_zero_kernel(TailPtrs ptrs, int n_ptrs, long long t_local, long long t_alloc,
                                                        int hq, int hkv, int d) {
  const long long tail = t_alloc - t_local;
  const long long uq = tail * hq * d / 8, ukv = tail * hkv * d / 8;
  const long long n = uq + (long long)(n_ptrs - 1) * ukv;
  for (long long e = blockIdx.x * (long long)blockDim.x + threadIdx.x; e < n; e += (long long)gridDim.x * blockDim.x) {
    uint16_t* base;
    long long u;
    if (e < uq) {
      base = ptrs.p[0] + t_local * hq * d;
      u = e;
    } else {
      const long long r = e - uq;
      const int which = 1 + (int)(r / ukv);
      base = ptrs.p[which] + t_local * hkv * d;
      u = r - (long long)(which - 1) * ukv;
    }
    reinterpret_cast<uint4*>(base)[u] = make_uint4(0, 0, 0, 0);
  }
}

// Whether the backward runs its dK/dV launch beside its dQ launch: only when
// the dQ launch is short (long ones measured slower with co-resident blocks).
bool bwd_forks(const cp_attn_meta* m, int hq) { return short_launches(m->sum.tiles_fwd[0] * hq, m->device); }

static unsigned grid_for(long long n, int per_block) {
  long long b = (n + per_block - 1) / per_block;
  if (b < 1) b = 1;
  return (unsigned)std::min<long long>(b, 8192);
}

}  // namespace cpattn

using namespace cpattn;

// The backward of both entry points. ws: the per-row planes (lse in exp2
// units, -D), cp_attn_workspace_bytes(.., 1) bytes, already checked by the
// caller; may_fork: whether short launches may run on a side stream.
static cp_attn_status bwd_run(const cp_attn_meta* m, const void* q, const void* const* k_shards,
                              const void* const* v_shards, const void* out, const float* lse, const void* dout,
                              int32_t hq, int32_t hkv, int32_t d, float softmax_scale, void* dq,
                              void* const* dk_parts, void* const* dv_parts, void* workspace, void* stream,
                              bool may_fork);

// Argument checks shared by both entry points (before any launch).
static cp_attn_status bwd_check(const cp_attn_meta* m, const void* q, const void* const* k_shards,
                                const void* const* v_shards, const void* out, const float* lse, const void* dout,
                                int32_t hq, int32_t hkv, int32_t d, float softmax_scale, int32_t causal, void* dq,
                                void* const* dk_parts, void* const* dv_parts) {
  if (!m) return fail(CP_ATTN_ERR_INVALID_ARG, "meta is NULL");
  if (!q || !k_shards || !v_shards || !out || !lse || !dout || !dq || !dk_parts || !dv_parts)
    return fail(CP_ATTN_ERR_INVALID_ARG, "NULL tensor argument");
  if (causal != 1) return fail(CP_ATTN_ERR_UNSUPPORTED, "only causal attention is supported");
  if (d != 64 && d != 128) return fail(CP_ATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return fail(CP_ATTN_ERR_INVALID_ARG, "hq must be a positive multiple of hkv");
  if (!(softmax_scale > 0.f) || !(softmax_scale < 1e30f))
    return fail(CP_ATTN_ERR_INVALID_ARG, "softmax_scale must be positive and finite");
  const int cp = m->cp;
  uintptr_t al = (uintptr_t)q | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dq;
  for (int s = 0; s < cp; ++s) {
    if (!k_shards[s] || !v_shards[s] || !dk_parts[s] || !dv_parts[s])
      return fail(CP_ATTN_ERR_INVALID_ARG, "NULL shard / part pointer");
    al |= (uintptr_t)k_shards[s] | (uintptr_t)v_shards[s] | (uintptr_t)dk_parts[s] | (uintptr_t)dv_parts[s];
  }
  if (al & 15) return fail(CP_ATTN_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != m->device)
    return fail(CP_ATTN_ERR_INVALID_ARG, "current device differs from the metadata's device");
  if ((long long)hq * d * 2 > (1ll << 20))
    return fail(CP_ATTN_ERR_UNSUPPORTED, "a row of all heads must stay within 1 MiB");
  return CP_ATTN_OK;
}

extern "C" cp_attn_status cp_attn_bwd(const cp_attn_meta* m, const void* q, const void* const* k_shards,
                                      const void* const* v_shards, const void* out, const float* lse,
                                      const void* dout, int32_t hq, int32_t hkv, int32_t d, float softmax_scale,
                                      int32_t causal, void* dq, void* const* dk_parts, void* const* dv_parts,
                                      void* workspace, size_t ws_bytes, void* stream) {
  set_error("");
  cp_attn_status rc = bwd_check(m, q, k_shards, v_shards, out, lse, dout, hq, hkv, d, softmax_scale, causal, dq,
                                dk_parts, dv_parts);
  if (rc != CP_ATTN_OK) return rc;
  const size_t need = cp_attn_workspace_bytes(m, hq, hkv, d, 1);
  if (!workspace || ws_bytes < need) return fail(CP_ATTN_ERR_WORKSPACE, "backward workspace missing or too small");
  if (((uintptr_t)workspace) & 255) return fail(CP_ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return bwd_run(m, q, k_shards, v_shards, out, lse, dout, hq, hkv, d, softmax_scale, dq, dk_parts, dv_parts,
                 workspace, stream, true);
}

static cp_attn_status bwd_run(const cp_attn_meta* m, const void* q, const void* const* k_shards,
                              const void* const* v_shards, const void* out, const float* lse, const void* dout,
                              int32_t hq, int32_t hkv, int32_t d, float softmax_scale, void* dq,
                              void* const* dk_parts, void* const* dv_parts, void* workspace, void* stream,
                              bool may_fork) {
  const int cp = m->cp;
  hipStream_t st = (hipStream_t)stream;
  const int tl = m->sum.t_local;
  cp_attn_status rc = CP_ATTN_OK;
  if (tl > 0) {
    const size_t l_al = (((size_t)tl * hq * sizeof(float)) + 255) & ~size_t(255);
    float* lse2 = (float*)workspace;
    float* negd = (float*)((char*)workspace + l_al);
    const int32_t* rowflags = m->d_tab + m->lay.rowflags;
    timing_begin(st, "bwd_pre");
    hipLaunchKernelGGL(bwd_pre_kernel, dim3(grid_for((long long)tl * hq * (d / 8), 256)), dim3(256), 0, st,
                       (const uint16_t*)dout, (const uint16_t*)out, lse, (long long)m->t_alloc, rowflags, lse2, negd,
                       tl, hq, d);
    timing_end(st);
    if ((rc = hip_check(hipGetLastError(), "bwd_pre launch")) != CP_ATTN_OK) return rc;
    BwdParams base{};
    base.q = (const uint16_t*)q;
    base.dout = (const uint16_t*)dout;
    base.lse2 = lse2;
    base.negd = negd;
    base.ld_ldv = tl;
    base.steps = m->d_tab + m->lay.steps;
    base.B = m->B;
    base.slot = m->d_tab + m->lay.cupl;
    base.items = m->d_tab + m->lay.fwd_tiles;  // the causal step's (step 0) query tiles
    base.hq = hq;
    base.hkv = hkv;
    base.group = hq / hkv;
    base.ld_q = (long long)hq * d;
    base.ld_kv = (long long)hkv * d;
    base.scale = softmax_scale;
    base.c_log2 = softmax_scale * LOG2E_F;
    base.dq = (uint16_t*)dq;
    const bool big = (long long)tl * hq * d * 2 >= (1ll << 31);  // local query tensors of 2 GiB or more
    // dK/dV of every ring step in one launch (each step writes its own part),
    // and dQ of every step in one launch (each block sums its rows' steps in
    // registers). The two launches are independent (both read what bwd_pre
    // wrote): short ones run concurrently, the dK/dV one on a side stream
    // forked from the caller's; long ones stay on one stream (co-resident
    // dK/dV and dQ blocks measured slower there).
    DkdvSteps ks{};
    DqSteps qs{};
    long long nkv = 0;
    for (int i = 0; i < cp; ++i) {
      const int s = m->sum.step_src[i];
      qs.k[i] = (const uint16_t*)k_shards[s];
      qs.v[i] = (const uint16_t*)v_shards[s];
      qs.kind[i] = m->sum.step_kind[i];
    }
    // the dK/dV launch dispatches the causal step's work items last: the
    // other steps' blocks all sweep the whole query range from its end, so
    // the ones running together read the same Q / dO tiles (shared in L2);
    // the causal step's sweeps have different lengths and would put them out
    // of step if its blocks came first
    for (int k = 0; k < cp; ++k) {
      const int i = (k + 1) % cp;  // steps 1 .. CP-1, then the causal step 0
      const int s = m->sum.step_src[i];
      const long long nb = m->sum.tiles_dkdv[i] * hkv;
      if (nb == 0) continue;
      const int j = ks.n++;
      ks.k[j] = qs.k[i];
      ks.v[j] = qs.v[i];
      ks.dk[j] = (uint16_t*)dk_parts[s];
      ks.dv[j] = (uint16_t*)dv_parts[s];
      ks.items[j] = m->d_tab + m->lay.dkdv_tiles + (int64_t)i * m->lay.dkdv_cap * 2;
      ks.step[j] = i;
      ks.kind[j] = m->sum.step_kind[i];
      ks.off[j] = (int)nkv;
      nkv += nb;
    }
    ks.off[ks.n] = (int)nkv;
    qs.n = cp;
    if (nkv > 0x7fffffffLL) return fail(CP_ATTN_ERR_UNSUPPORTED, "too many work items");
    const long long nq = m->sum.tiles_fwd[0] * hq;
    const bool fork = may_fork && bwd_forks(m, hq);
    SideSet* side = nullptr;
    hipStream_t sk = st;
    if (fork && nkv > 0) {
      if ((rc = side_set(m->device, &side)) != CP_ATTN_OK) return rc;
      sk = side->s[0];
      if ((rc = fork_to(side, st, 1)) != CP_ATTN_OK) return rc;
    }
    cp_attn_status lrc = CP_ATTN_OK;  // launch errors wait for the join
    if (nkv > 0) {
      timing_begin(sk, "bwd_dkdv");
      if (d == 128) {
        if (big)
          hipLaunchKernelGGL((bwd_dkdv_kernel<128, true>), dim3((unsigned)nkv), dim3(BLOCK_THREADS), 0, sk, base, ks);
        else
          hipLaunchKernelGGL((bwd_dkdv_kernel<128, false>), dim3((unsigned)nkv), dim3(BLOCK_THREADS), 0, sk, base, ks);
      } else {
        if (big)
          hipLaunchKernelGGL((bwd_dkdv_kernel<64, true>), dim3((unsigned)nkv), dim3(BLOCK_THREADS), 0, sk, base, ks);
        else
          hipLaunchKernelGGL((bwd_dkdv_kernel<64, false>), dim3((unsigned)nkv), dim3(BLOCK_THREADS), 0, sk, base, ks);
      }
      timing_end(sk);
      lrc = hip_check(hipGetLastError(), "bwd_dkdv launch");
    }
    if (lrc == CP_ATTN_OK && nq > 0) {
      if (nq > 0x7fffffffLL) lrc = fail(CP_ATTN_ERR_UNSUPPORTED, "too many work items");
      else {
        timing_begin(st, "bwd_dq");
        if (d == 128)
          hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3((unsigned)nq), dim3(BLOCK_THREADS), 0, st, base, qs);
        else
          hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3((unsigned)nq), dim3(BLOCK_THREADS), 0, st, base, qs);
        timing_end(st);
        lrc = hip_check(hipGetLastError(), "bwd_dq launch");
      }
    }
    if (side && (rc = join_from(side, st, 1)) != CP_ATTN_OK) return rc;
    if (lrc != CP_ATTN_OK) return lrc;
    if (m->sum.valid_rows < tl) {
      timing_begin(st, "dq_pad_rows");
      hipLaunchKernelGGL(dq_pad_rows_kernel, dim3(grid_for((long long)tl * hq * d / 8, 256)), dim3(256), 0, st,
                         rowflags, (uint16_t*)dq, tl, hq, d);
      timing_end(st);
      if ((rc = hip_check(hipGetLastError(), "dq_pad_rows launch")) != CP_ATTN_OK) return rc;
    }
  }
  if (m->sum.has_tail) {
    TailPtrs tp{};
    tp.p[0] = (uint16_t*)dq;
    for (int s = 0; s < cp; ++s) {
      tp.p[1 + s] = (uint16_t*)dk_parts[s];
      tp.p[1 + cp + s] = (uint16_t*)dv_parts[s];
    }
    const long long tail = m->t_alloc - tl;
    const long long n = tail * hq * d / 8 + (long long)2 * cp * tail * hkv * d / 8;
    timing_begin(st, "tail_zero");
    hipLaunchKernelGGL(tail_zero_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, tp, 1 + 2 * cp, (long long)tl,
                       (long long)m->t_alloc, hq, hkv, d);
    timing_end(st);
    rc = hip_check(hipGetLastError(), "tail_zero launch");
  }
  return rc;
}

// ------------------------------------------------ allocation-free backward
// cp_attn_bwd_noalloc takes its per-row planes (the only scratch the
// backward needs: lse in exp2 units and -D, 8 * hq * T_local bytes) from a
// fixed device array instead of a caller's workspace, for callers that
// cannot allocate. Each GPU holds its own copy of the array for the life of
// the process; its device address is looked up once per device (the array's
// name in host code is a host-side stand-in, not a device address) and only
// that address is handed to kernels. Every call on one GPU uses the same
// array: calls that overlap on one GPU race. Nothing in it has to start at
// zero (bwd_pre writes every row it holds before the other kernels read it).
namespace cpattn {
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(32) << 20;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];
static std::atomic<void*> g_scratch_ptr[64];
static std::mutex g_scratch_mu;

// The array's address on the current device (looked up on first use).
static cp_attn_status scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= 64) return fail(CP_ATTN_ERR_INVALID_ARG, "device index out of range");
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      cp_attn_status rc = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
      if (rc != CP_ATTN_OK) return rc;
      if (!p) return fail(CP_ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return CP_ATTN_OK;
}
}  // namespace cpattn

extern "C" cp_attn_status cp_attn_bwd_noalloc(const cp_attn_meta* m, const void* q, const void* const* k_shards,
                                              const void* const* v_shards, const void* out, const float* lse,
                                              const void* dout, int32_t hq, int32_t hkv, int32_t d,
                                              float softmax_scale, int32_t causal, void* dq, void* const* dk_parts,
                                              void* const* dv_parts, void* stream) {
  set_error("");
  cp_attn_status rc = bwd_check(m, q, k_shards, v_shards, out, lse, dout, hq, hkv, d, softmax_scale, causal, dq,
                                dk_parts, dv_parts);
  if (rc != CP_ATTN_OK) return rc;
  const size_t need = cp_attn_workspace_bytes(m, hq, hkv, d, 1);
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(CP_ATTN_ERR_WORKSPACE, "share too large for the allocation-free backward: needs " +
                                           std::to_string(need) + " bytes of scratch, the fixed array holds " +
                                           std::to_string(NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if ((rc = scratch_on(m->device, &ws)) != CP_ATTN_OK) return rc;
  return bwd_run(m, q, k_shards, v_shards, out, lse, dout, hq, hkv, d, softmax_scale, dq, dk_parts, dv_parts, ws,
                 stream, false);
}
