// Device helpers shared by the attention kernels (gfx950 / CDNA4 only).
//
// MFMA used throughout: v_mfma_f32_32x32x16_bf16 (one wavefront of 64 lanes).
// Operand layouts, with lane = 32 * g + i (g = 0/1, i = 0..31):
//   A (32 x 16, row-major M x K): lane holds row i, k = 8g .. 8g+7
//   B (16 x 32, K x N):          lane holds column i, k = 8g .. 8g+7
//   C (32 x 32 fp32, 16 values): lane holds column i, rows
//                                8*(j/4) + 4*g + (j%4), j = 0..15
// Because the contraction runs over k, any permutation of k applied to both
// A and B leaves the product unchanged. The kernels use this to feed a C
// fragment (lane = one column, 16 rows) straight back as a B operand: the
// eight values j = 8h .. 8h+7 of a C fragment are the "k = 8g..8g+7" of the
// 16-wide slice h, which pairs with A rows read at the matching positions
// 16h + 4g + {0,1,2,3} and 16h + 8 + 4g + {0,1,2,3}.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace cpattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float NEG_INF_F = -__builtin_huge_valf();
constexpr float LOG2E_F = 1.4426950408889634f;

__device__ __forceinline__ f32x16_t mfma32x32x16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int j = 0; j < 16; ++j) z[j] = 0.f;
  return z;
}

// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint2& lo, const uint2& hi) {
  uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return __builtin_bit_cast(bf16x8_t, u);
}

// Eight consecutive fp32 values of a C fragment -> bf16 B operand.
__device__ __forceinline__ bf16x8_t pack8_bf16(const f32x16_t& c, int j0) {
  uint4 u;
  u.x = pack2_bf16(c[j0 + 0], c[j0 + 1]);
  u.y = pack2_bf16(c[j0 + 2], c[j0 + 3]);
  u.z = pack2_bf16(c[j0 + 4], c[j0 + 5]);
  u.w = pack2_bf16(c[j0 + 6], c[j0 + 7]);
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lanes i and i ^ 32 combined without an LDS round trip: v_permlane32_swap
// applied to (x, x) hands every lane x of lane (i & 31) and of lane
// (i & 31) + 32.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// bf16 halves of two dwords -> one dword (lo from a, hi from b), selected half
__device__ __forceinline__ uint32_t pick_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pick_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ __forceinline__ uint32_t u4_get(const uint4& u, int w) {
  return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

// Transpose a 4 (rows) x 8 (cols) bf16 block held as four 16-byte rows into
// eight 4-element columns, written as 8-byte LDS stores to dst + e * stride.
__device__ __forceinline__ void store_transposed_4x8(uint16_t* dst, int stride, const uint4& r0, const uint4& r1,
                                                     const uint4& r2, const uint4& r3) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t a0 = u4_get(r0, w), a1 = u4_get(r1, w), a2 = u4_get(r2, w), a3 = u4_get(r3, w);
    uint2 ev = make_uint2(pick_lo(a0, a1), pick_lo(a2, a3));
    uint2 od = make_uint2(pick_hi(a0, a1), pick_hi(a2, a3));
    *reinterpret_cast<uint2*>(dst + (2 * w) * stride) = ev;
    *reinterpret_cast<uint2*>(dst + (2 * w + 1) * stride) = od;
  }
}

// Output rows through LDS. In the MFMA accumulator layout a lane holds
// elements d = 32 md + 8 jj + 4 g + e (e = 0..3) of one row; parking them in
// a padded row-major staging tile lets every global store write 16 bytes of
// a whole row (D * 2 / 16 lanes per row) instead of 8 bytes in each of 32
// rows. stage_row_bf16 writes one lane's share of `row` (scaled by mul);
// store_rows copies staging rows [0, n) to dst rows (ld elements apart)
// with every thread of the block.
template <int D>
__device__ __forceinline__ void stage_row_bf16(char* row, int g, const f32x16_t (&v)[D / 32], float mul) {
#pragma unroll
  for (int md = 0; md < D / 32; ++md)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint2 pk;
      pk.x = pack2_bf16(v[md][4 * jj] * mul, v[md][4 * jj + 1] * mul);
      pk.y = pack2_bf16(v[md][4 * jj + 2] * mul, v[md][4 * jj + 3] * mul);
      *reinterpret_cast<uint2*>(row + (md * 32 + jj * 8 + g * 4) * 2) = pk;
    }
}

template <int D, int PITCH, int THREADS>
__device__ __forceinline__ void store_rows(const char* stage, int n, uint16_t* dst, long long ld, int tid) {
  constexpr int UPR = D * 2 / 16;
  for (int u = tid; u < n * UPR; u += THREADS) {
    const int r = u / UPR, c = u - r * UPR;
    *reinterpret_cast<uint4*>(dst + (long long)r * ld + c * 8) = *reinterpret_cast<const uint4*>(stage + r * PITCH + c * 16);
  }
}

// Block -> (work item, head). When the head count is a multiple of the 8
// XCDs, the blocks that land on one XCD (consecutive ids are dealt to the
// XCDs round-robin) take a contiguous run of heads, so a GQA group's K/V stay
// in one XCD's L2.
__device__ __forceinline__ void map_block(int bid, int nheads, int& item, int& head) {
  if ((nheads & 7) == 0) {
    const int per = nheads >> 3;
    const int xcd = bid & 7;
    const int r = bid >> 3;
    head = xcd * per + (r % per);
    item = r / per;
  } else {
    item = bid / nheads;
    head = bid - item * nheads;
  }
}

// Copy `units` 16-byte units from src to dst with the 64 lanes of a
// wavefront, four loads in flight per lane before their stores; the data is
// touched once, so both sides bypass cache retention (non-temporal).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void wave_copy(const uint4* __restrict__ src_, uint4* __restrict__ dst_, int units, int lane) {
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(src_);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(dst_);
  for (int base = 0; base < units; base += 256) {
    u32x4_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = base + i * 64 + lane;
      if (u < units) v[i] = __builtin_nontemporal_load(src + u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = base + i * 64 + lane;
      if (u < units) __builtin_nontemporal_store(v[i], dst + u);
    }
  }
}

// ---------------------------------------------------------------- LDS tiles
// Row-major tiles (rows x D bf16) live in LDS with padded rows. gfx950's LDS
// has 64 banks of 4 bytes; a b128 read serves 16 lanes per cycle and the
// transposing ds_read_b64_tr_b16 serves 32 lanes per cycle. Row strides:
//  * tiles read by b128 row reads (16 lanes = one 16-byte unit of 16
//    consecutive rows), alone or together with transposing reads: 304 bytes
//    (D = 128) or 144 (D = 64) - conflict-free for the row reads;
//  * tiles read only by transposing reads (32 lanes take 64 consecutive bytes
//    of 4 rows): 320 bytes (D = 128) or 192 (D = 64) - conflict-free for 4
//    consecutive rows.
// A transposing read of 4 consecutive rows 304 (144) bytes apart hits each
// bank twice (measured: 4.1 instead of 2.3 cycles per instruction per CU).
// Tiles read both ways therefore store their rows permuted inside each
// 16-row block (perm_row below): the 4 logical rows a transposing read takes
// then sit 4 physical rows apart, 4 x 304 (144) bytes = 16 x odd banks, which
// is conflict-free, and the 16 rows a row read takes are still 16 distinct
// rows of one block. Padding and the permutation keep every address linear in
// the unrolled loop indices (only the per-lane base changes), so the compiler
// folds them into instruction offsets; an XOR swizzle that removed both kinds
// of conflict measured slower for its extra address arithmetic.
// Physical row of logical row r in a permuted tile: within each 16-row block
// (r = 16 b + 4 a + c) row 16 b + 4 c + a, a 4 x 4 transpose and its own
// inverse.
__host__ __device__ constexpr int perm_row(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

template <int D, bool TR_ONLY>
__host__ __device__ constexpr int tile_rowb() { return TR_ONLY ? (D == 128 ? 320 : 192) : (D == 128 ? 304 : 144); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// A double buffer's index as a compile-time constant: kernels that name
// each buffer's LDS array statically let the compiler see that reads of one
// buffer cannot touch the other, whose copy is in flight, so it does not
// wait for that copy before them (with one array indexed by the buffer
// number it must).
template <int B>
using Buf = std::integral_constant<int, B>;

// Direct global->LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane l of the wavefront writes LDS bytes [chunk + 16 l, chunk + 16 l + 16).
// Offsets at or past the resource's num_records read as zeros.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds_chunk, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds_chunk, 16, voffset, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr int OOB_OFFSET = 0x7ffffff0;  // any offset past num_records reads zeros

// Copy plan of one tile of ROWS x D bf16 (global rows ld_bytes apart) into a
// padded LDS tile. The tile is filled as a linear run of 16-byte units in
// 1 KB chunks (64 lanes x 16 bytes) dealt round-robin to the block's NW
// wavefronts; the LDS tile spans whole chunks (BYTES), so lanes past the last
// row only fill spare bytes with zeros. A lane's global offset within a tile
// depends on the lane alone and is computed once (row padding units get an
// offset past any buffer's end and load zeros). Each copy takes a buffer
// resource whose base is the tile's first row and whose size ends at the
// range's end, so rows past the range load zeros.
template <int D, bool TR_ONLY, int ROWS, int NW, bool PERM = false>
struct TileCopy {
  static_assert(!PERM || ROWS % 16 == 0, "permuted tiles hold whole 16-row blocks");
  static constexpr int SU = tile_rowb<D, TR_ONLY>() / 16;  // units per padded row
  static constexpr int UPR = D * 2 / 16;                   // units per data row
  static constexpr int UNITS = ROWS * SU;
  static constexpr int CHUNKS = (UNITS + 63) / 64;
  static constexpr int PER_WAVE = (CHUNKS + NW - 1) / NW;
  static constexpr int BYTES = CHUNKS * 1024;
  int voff[PER_WAVE];

  __device__ __forceinline__ void init(int ld_bytes, int wave, int lane) {
#pragma unroll
    for (int cc = 0; cc < PER_WAVE; ++cc) {
      const int u = (cc * NW + wave) * 64 + lane;
      const int row = u / SU, unit = u % SU;
      const int src = PERM ? perm_row(row) : row;  // perm_row is an involution
      voff[cc] = (unit < UPR && u < UNITS) ? src * ld_bytes + unit * 16 : OOB_OFFSET;
    }
  }
  __device__ __forceinline__ void copy(__amdgpu_buffer_rsrc_t rsrc, void* lds_tile, int wave) const {
#pragma unroll
    for (int cc = 0; cc < PER_WAVE; ++cc) {
      const int c = cc * NW + wave;
      if (CHUNKS % NW == 0 || c < CHUNKS) load_lds16(rsrc, reinterpret_cast<char*>(lds_tile) + c * 1024, voff[cc]);
    }
  }
};

// Buffer resource over [base + off_bytes, base + end_bytes): rows from
// off_bytes on, nothing once off_bytes passes end_bytes. The base is rebased
// on off_bytes in 64-bit arithmetic, so tensors of any size can be
// addressed; the record count is capped at RSRC_CAP (far more than any tile
// reads), which keeps OOB_OFFSET out of range.
constexpr long long RSRC_CAP = 1ll << 30;
// the same with 32-bit offsets, for ranges known to stay below 2 GiB
// (cheaper scalar arithmetic on the per-iteration path)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_from32(const void* base, int off_bytes, int end_bytes) {
  const int n = end_bytes - off_bytes;
  return make_rsrc(reinterpret_cast<const char*>(base) + off_bytes, n > 0 ? n : 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_from(const void* base, long long off_bytes, long long end_bytes) {
  const long long n = end_bytes - off_bytes;
  return make_rsrc(reinterpret_cast<const char*>(base) + off_bytes, n <= 0 ? 0 : (n < RSRC_CAP ? n : RSRC_CAP));
}

// b128 read of 16-byte unit `unit` of logical row `row` (tiles with row
// reads; PERM for tiles stored with permuted rows).
template <int D, bool PERM = false>
__device__ __forceinline__ bf16x8_t lds_read_row(const uint16_t* tile, int row, int unit) {
  const int prow = PERM ? perm_row(row) : row;
  return as_bf16x8(*reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(tile) + prow * tile_rowb<D, false>() +
                                                   unit * 16));
}

// Transposed operand (ds_read_b64_tr_b16) for the 32-wide MFMA A operand
// with k running over tile rows: lane (32 g + i) receives column col0 + i of
// rows k0 + 4 g + {0..3} and k0 + 8 + 4 g + {0..3} (col0 a multiple of 32, k0
// a multiple of 16). Within each 16-lane group, lane j supplies the address
// of row (first + j / 4), columns 4 (j % 4) .. +3 of its 16-column half; the
// hardware hands lane j column j of those four rows.
// In a permuted tile (PERM) logical rows k0 + 4 g + (i / 4) and k0 + 8 + 4 g +
// (i / 4) sit at physical rows k0 + 4 (i / 4) + g and 2 rows further on.
template <int D, bool TR_ONLY, bool PERM = false, bool OPAQUE = TR_ONLY>
__device__ __forceinline__ bf16x8_t lds_read_tr(const uint16_t* tile, int k0, int col0, int lane) {
  static_assert(!(PERM && TR_ONLY), "permuted tiles use the row-read stride");
  constexpr int ROWB = tile_rowb<D, TR_ONLY>();
  const int i = lane & 15, h = (lane >> 4) & 1, g = lane >> 5;
  const char* base;
  if constexpr (OPAQUE) {
    // the lane's offset as one opaque value (computed once) plus a constant
    // per read: each address is then a short chain of additions from the
    // tile, short enough for the compiler to see which LDS array the read
    // touches, so it waits only for copies into that array (the forward's
    // V tiles and dQ's K tiles; measured neutral to slower on dK/dV's)
    int lane_off = (PERM ? 4 * (i >> 2) + g : 4 * g + (i >> 2)) * ROWB + (16 * h + 4 * (i & 3)) * 2;
    __asm__("" : "+v"(lane_off));
    base = reinterpret_cast<const char*>(tile) + lane_off + (k0 * ROWB + col0 * 2);
  } else {
    const int col = col0 + 16 * h + 4 * (i & 3);
    const int r0 = PERM ? k0 + 4 * (i >> 2) + g : k0 + 4 * g + (i >> 2);
    base = reinterpret_cast<const char*>(tile) + r0 * ROWB + col * 2;
  }
  i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(base));
  i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(base + (PERM ? 2 : 8) * ROWB));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

}  // namespace cpattn
