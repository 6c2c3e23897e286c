// Device helpers shared by the attention kernels (gfx950 / CDNA4, wave64).
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_bf16), for lane l, half h = l / 32:
//   A (32 x 16):  lane l holds A[l % 32][8h .. 8h + 7]        (8 bf16 = one 16-byte register quad)
//   B (16 x 32):  lane l holds B[8h .. 8h + 7][l % 32]
//   C (32 x 32):  lane l holds C[8 (r / 4) + 4h + (r % 4)][l % 32] in accumulator register r = 0..15
// The contraction index k only has to agree between A and B, so each kernel maps k slots to
// keys or queries in whatever order makes the operands it already holds line up.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaskBlock = 128;
constexpr int kMaxMaskBlocks = 2048;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
}

// ---------------------------------------------------------------------------------------------
// LDS tiles: rows of D bf16 (D * 2 bytes, a multiple of 128 bytes), with the 16-byte chunk index
// inside a row XOR-swizzled by f(row) = 2 (row % 4) + (row / 4) % 2.
//  * 16-byte row reads (ds_read_b128, 8 lanes per LDS cycle reading 8 consecutive rows at the
//    same column) hit 8 distinct chunk slots: f takes 8 distinct values over 8 consecutive rows.
//  * transposed reads (ds_read_b64_tr_b16: 16 lanes read 4 consecutive rows x 32 bytes) hit
//    8 distinct slots: f(row) / 2 takes 4 distinct values over 4 consecutive rows.
//  * 16-byte writes of 8 consecutive chunks of one row are a permutation of that row's slots.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

// byte offset of element (row, col) in a tile with D columns; col must be a multiple of 4
template <int D>
__device__ __forceinline__ int lds_off(int row, int col) {
  return row * (D * 2) + ((((col >> 3) ^ swz(row))) << 4) + ((col & 7) << 1);
}

template <int D>
__device__ __forceinline__ bf16x8 lds_row8(const char* tile, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(tile + lds_off<D>(row, col));
}

// Transposed read: returns, for lane l (16-lane group g = l / 16, i = l % 16), the 4 values
// tile[row_t][col0 + i] for t = 0..3, where lane j of the group addresses tile[row_{j/4}][col0 + 4 (j%4)].
// Each lane passes its own address; the hardware exchanges the 16-bit elements within the group.
__device__ __forceinline__ s16x4 lds_tr4(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

__device__ __forceinline__ bf16x8 join8(s16x4 a, s16x4 b) {
  s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// A operand (rows = 32 columns of a row-major LDS tile, k slots = 8 tile rows) read transposed:
// lane l (half h, c = l % 32) receives tile[row(h, e)][col_base + c] for e = 0..7 with
// row(h, 4u + t) = row_base + 8u + 4h + t.  This matches the k-slot order of an MFMA C
// accumulator whose rows 16m + 8u + 4h + t sit in registers 8m + 4u + t.
template <int D>
__device__ __forceinline__ bf16x8 lds_tr_operand(const char* tile, int row_base, int col_base, int lane) {
  const int h = lane >> 5, g = (lane >> 4) & 1, j = lane & 15;
  const int col = col_base + 16 * g + 4 * (j & 3);
  const int r0 = row_base + 4 * h + (j >> 2);
  s16x4 lo = lds_tr4(tile + lds_off<D>(r0, col));
  s16x4 hi = lds_tr4(tile + lds_off<D>(r0 + 8, col));
  return join8(lo, hi);
}

// ---------------------------------------------------------------------------------------------
// wave64 cross-half reductions: lanes l and l ^ 32 hold partial results for the same query.
// v_permlane32_swap exchanges the upper half of its first operand with the lower half of its
// second; called with (x, x) every lane ends up holding both its own value and its partner's.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------------------
// Tile scheduler decode.  The grid is one workgroup per (b*h, tile).  Consecutive workgroup ids
// are dispatched round-robin over the 8 XCDs (each with its own L2); when the item count and
// B*H are multiples of 8, ids are remapped so that every XCD works through B*H/8 whole heads,
// keeping a head's K/V (or Q/dO) re-reads inside one L2.  Within a head group the heaviest tiles
// come first (the causal triangle gives tile t of the query side t + 1 units of work).
// ---------------------------------------------------------------------------------------------
struct Sched {
  int ntiles;  // tiles per head
  int group;   // heads per XCD group (divides B*H)
  int remap;   // 1: XCD-aware remap active
  int heavy_last_tile;  // 1: tile ntiles-1 is the heaviest (query side); 0: tile 0 is
};

__device__ __forceinline__ void sched_decode(const Sched& s, int total, int& bh, int& tile) {
  int w = blockIdx.x;
  if (s.remap) w = (w & 7) * (total >> 3) + (w >> 3);
  const int per = s.group * s.ntiles;
  const int hg = w / per;
  const int r = w - hg * per;
  const int t = r / s.group;
  tile = s.heavy_last_tile ? (s.ntiles - 1 - t) : t;
  bh = hg * s.group + (r - t * s.group);
}

// Builds, in LDS, the ascending list of mask blocks J with block_mask[I][J] != 0 (row mode) or
// block_mask[J][I] != 0 (column mode), restricted to J in [lo, hi).  Run by one whole wave.
__device__ __forceinline__ int build_block_list(const uint8_t* mask, int nb, int I, bool column, int lo, int hi,
                                                unsigned short* list, int lane) {
  int cnt = 0;
  for (int base = lo; base < hi; base += 64) {
    const int J = base + lane;
    bool on = false;
    if (J < hi) on = (column ? mask[(size_t)J * nb + I] : mask[(size_t)I * nb + J]) != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
    if (on) list[cnt + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] = (unsigned short)J;
    cnt += __builtin_popcountll(bal);
  }
  return cnt;
}

}  // namespace fa
