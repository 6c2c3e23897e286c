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

// XOR a per-dword mask into 8 packed bf16: with 0x80008000 every element changes sign (exact,
// including zeros and NaN), with 0 nothing changes
__device__ __forceinline__ bf16x8 xor_sign(bf16x8 x, uint32_t m) {
  uint4 u = __builtin_bit_cast(uint4, x);
  u.x ^= m;
  u.y ^= m;
  u.z ^= m;
  u.w ^= m;
  return __builtin_bit_cast(bf16x8, u);
}

// ---------------------------------------------------------------------------------------------
// LDS operand reads.  Row operands use 16-byte ds_read_b128 (LDS serves 16 lanes per pass over a
// 256-byte bank window); operands that need the contraction index inside a lane use the 8-byte
// transposing ds_read_b64_tr_b16, which a conflict-free probe on gfx950 measured at about 0.7 of
// the row-read bandwidth.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 lds_b128(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Transposing 8-byte LDS read: within each 16-lane group, lane i receives element i % 4 of the
// 8 bytes addressed by lanes 4t + i / 4 (t = 0..3), i.e. a 4 x 4 block transpose per 4 lanes.
__device__ __forceinline__ s16x4 lds_tr4(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}
__device__ __forceinline__ bf16x8 join8(s16x4 a, s16x4 b) {
  s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Row order used for A operands whose MFMA result feeds a later contraction: reading row
// perm32(i) of a 32-row block into A-row i swaps bits 2 and 3 of the row index.  The C
// accumulator then holds, in registers 8m .. 8m+7 of lane half h, rows 16m + 8h + 0..7 of the
// block (consecutive), which is exactly one 8-element k-slot group of a 32x32x16 operand.
__device__ __forceinline__ constexpr int perm32(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}
// block row held by accumulator register r of lane half h after that permutation
__device__ __forceinline__ constexpr int acc_row(int r, int h) {
  return 16 * (r >> 3) + 8 * h + 4 * ((r >> 2) & 1) + (r & 3);
}

// Global reads through buffer resources: the hardware range check returns zero for any byte
// offset at or past num_records, which covers the ragged last tile of a head without branches.
// A resource spans one head's [N, d] slice (at most 2^31 - 1 bytes, checked on the host).
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcFlags = 0x00020000;  // raw 32-bit data, no format conversion

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcFlags);
}

// ---------------------------------------------------------------------------------------------
// Asynchronous global -> LDS copies (buffer_load_dwordx4 ... lds): no registers, no VALU.  One
// instruction moves 64 lanes x 16 bytes into 1 KB of LDS, lane i landing at base + 16 i; the
// global address of each lane is free, so a tile lands in whatever 16-byte-chunk order the
// reads want.  The issuing wave waits for its copies with vmcnt(0); a barrier then publishes
// the tile to the other waves.
//
// DmaTile<R, D, SW> stages R rows x D bf16 (R*D/8 16-byte chunks, a multiple of 256) with the
// chunk order "physical chunk = logical chunk ^ SW(row)".
// ---------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* LdsPtr;

__device__ __forceinline__ void dma16(const Rsrc& r, void* lds_block, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)lds_block, 16, voff, soff, 0, 0);
}  // soff stays 0 in this library: the range check does not cover it
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// workgroup barrier that waits for this wave's LDS operations only (copies into LDS still in
// flight stay in flight), and that the compiler moves no memory access across
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// wait until at most N of this wave's vector-memory instructions (copies included) are in
// flight; they complete in issue order, so everything issued before the last N has landed
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte chunk swizzle (row = tile row, D = row length in bf16), free of LDS bank conflicts
// for both read patterns (64 banks x 4 bytes = one 256-byte window of 16 chunk slots):
//  row reads (16 bytes per lane, 16 lanes per cycle): the lanes read one logical chunk of 16
//             rows, so f must be a bijection on rows 0..15 (d = 64: two rows share a window,
//             so on the 8 even and on the 8 odd rows);
//  transposed reads (8 bytes per lane, 32 lanes per cycle): the lanes read 4 logical chunks
//             (an aligned group of 4) of 4 consecutive rows 4u .. 4u+3, so the rows sharing a
//             window must move the group to different aligned slots: f & 12 distinct across
//             them (d = 64: bit 2 of f distinct between rows 4u and 4u+2, 4u+1 and 4u+3).
template <int D>
__device__ __forceinline__ constexpr int sw_dual(int row) {
  return D >= 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Checking build (-DFA_CHECK): before a wave starts an asynchronous copy into LDS it fills the
// 16-byte chunks the copy will land in with NaN (0xFF bytes: NaN in bf16 and in E4M3), so that a
// read of the tile that runs ahead of the copy (a missing wait or barrier) carries NaN into the
// results.  `dst` is the first of `n` 1 KB blocks this wave fills, lane i at offset 16 i.
__device__ __forceinline__ void lds_sentinel(char* dst, int n, int lane) {
#ifdef FA_CHECK
  const uint4 nan4 = make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
  for (int i = 0; i < n; ++i) *reinterpret_cast<uint4*>(dst + 1024 * i + 16 * lane) = nan4;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#else
  (void)dst;
  (void)n;
  (void)lane;
#endif
}

template <int R, int D, int NW = 4>
struct DmaTile {
  static constexpr int CPR = D / 8;
  static constexpr int BYTES = R * D * 2;
  static constexpr int CH = R * CPR / (64 * NW);  // instructions per wave (NW waves)
  static_assert(CH >= 1 && (R * CPR) % (64 * NW) == 0, "tile too small for the waves");
  __device__ static constexpr int sw(int row) { return sw_dual<D>(row); }
  // byte offset in the tile of the 16-byte chunk holding (row, col), col a multiple of 8
  __device__ static constexpr int off(int row, int col) { return row * D * 2 + (((col >> 3) ^ sw(row)) << 4); }
  // byte offset of (row, col) for a transposed 8-byte read, col a multiple of 4
  __device__ static constexpr int off4(int row, int col) { return off(row, col) + (col & 7) * 2; }
  int voff[CH];  // per-lane global byte offsets relative to the tile's first row
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int slot = 64 * (CH * w + i) + lane;
      const int row = slot / CPR, pchunk = slot % CPR;
      voff[i] = (row * D + ((pchunk ^ sw(row)) << 3)) * 2;
    }
  }
  // enqueue the copy of rows [row0, row0 + R) of `head` (N rows) into `tile`; rows >= N read
  // as zero.  The resource starts at row0 and spans only rows row0 .. N-1, so the hardware
  // range check (which covers the per-lane offset) does the clipping.
  __device__ __forceinline__ void issue(const __bf16* head, int N, char* tile, int row0, int w) const {
    lds_sentinel(tile + 1024 * CH * w, CH, __lane_id());
    const Rsrc r = make_rsrc(head + (size_t)row0 * D, max(N - row0, 0) * D * 2);
#pragma unroll
    for (int i = 0; i < CH; ++i) dma16(r, tile + 1024 * (CH * w + i), voff[i], 0);
  }
};

// maximum that propagates NaN (IEEE maximum): unlike fmaxf it needs no canonicalising moves of
// its operands, and three of them fuse into one v_maximum3_f32
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// ---------------------------------------------------------------------------------------------
// wave64 cross-half reductions: lanes l and l ^ 32 hold partial results for the same query.
// v_permlane32_swap exchanges the upper half of its first operand with the lower half of its
// second; called with (x, x) every lane ends up holding both its own value and its partner's.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// DPP row broadcast (gfx90a and later): every lane receives the value of lane k of its own row of
// 16 lanes.  k must be a constant after inlining and unrolling (the switch then folds away).
template <int K>
__device__ __forceinline__ float row_bcast_k(float v) {
  static_assert(K >= 0 && K < 16, "lane within a row of 16");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + K, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_bcast(float v, int k) {
  switch (k) {
    case 0: return row_bcast_k<0>(v);
    case 1: return row_bcast_k<1>(v);
    case 2: return row_bcast_k<2>(v);
    case 3: return row_bcast_k<3>(v);
    case 4: return row_bcast_k<4>(v);
    case 5: return row_bcast_k<5>(v);
    case 6: return row_bcast_k<6>(v);
    case 7: return row_bcast_k<7>(v);
    case 8: return row_bcast_k<8>(v);
    case 9: return row_bcast_k<9>(v);
    case 10: return row_bcast_k<10>(v);
    case 11: return row_bcast_k<11>(v);
    case 12: return row_bcast_k<12>(v);
    case 13: return row_bcast_k<13>(v);
    case 14: return row_bcast_k<14>(v);
    default: return row_bcast_k<15>(v);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Q^T operand of one lane held in registers: features 16 c + 8 h .. 16 c + 8 h + 7 of query row
// qrow for every 16-wide chunk c, the sign of the scale folded in (xor_sign).  Rows past N load
// row N - 1 and are zeroed after, so the loads have no branch around them and are all in flight
// together (a branch per chunk made each wait for the one before).
template <int DC>
__device__ __forceinline__ void load_qt_operand(const __bf16* __restrict__ Q, int qrow, int N, int h, uint32_t qsign,
                                                bf16x8 (&qreg)[DC]) {
  const __bf16* row = Q + (size_t)min(qrow, N - 1) * (16 * DC);
#pragma unroll
  for (int c = 0; c < DC; ++c) qreg[c] = *reinterpret_cast<const bf16x8*>(row + 16 * c + 8 * h);
  const bool live = qrow < N;
#pragma unroll
  for (int c = 0; c < DC; ++c) qreg[c] = live ? xor_sign(qreg[c], qsign) : zero_bf16x8();
}

// ---------------------------------------------------------------------------------------------
// Tile scheduler decode.  The grid is one workgroup per (b*h, tile).  Consecutive workgroup ids
// are dispatched round-robin over the 8 XCDs (each with its own L2); when B*H is a multiple of 8,
// ids are remapped so that every XCD works through B*H/8 whole heads, keeping a head's K/V (or
// Q/dO) re-reads inside one L2.  Within an XCD the order is either
//  - tile-major: tile level by tile level, heaviest level first, all the XCD's heads at each level
//    (best balance when a head has few tiles: the causal triangle gives query tile t t + 1 units
//    of work, so the long tiles must start first), or
//  - head-major: one head after another, each heaviest tile first, so that the workgroups in
//    flight on an XCD stream the same head's K/V tiles at about the same time and share them in
//    L2 (always when a head's tiles carry equal work; with the causal triangle or a block mask,
//    once a head has enough tiles to fill the XCD's slots, where the late start of the last
//    head's long tiles is a small tail; see make_sched).
// ---------------------------------------------------------------------------------------------
struct Sched {
  int ntiles;      // tiles per head
  int group;       // heads per XCD group (divides B*H)
  int remap;       // 1: XCD-aware remap active
  int head_major;  // 1: head-major order inside a group (needs remap)
  int heavy_last_tile;  // 1: tile ntiles-1 is the heaviest (query side); 0: tile 0 is
  int slots;       // workgroups resident per XCD when a kernel alternates its key direction by
                   // cohort (sched_descending), else 0
};

__device__ __forceinline__ void sched_decode(const Sched& s, int total, int& bh, int& tile) {
  int w = blockIdx.x;
  if (s.remap) w = (w & 7) * (total >> 3) + (w >> 3);
  const int per = s.group * s.ntiles;
  const int hg = w / per;
  const int r = w - hg * per;
  int t, hh;
  if (s.head_major) {
    hh = r / s.ntiles;
    t = r - hh * s.ntiles;
  } else {
    t = r / s.group;
    hh = r - t * s.group;
  }
  tile = s.heavy_last_tile ? (s.ntiles - 1 - t) : t;
  bh = hg * s.group + hh;
}

// Key direction of a causal query tile under head-major order.  The XCD's slots fill with the
// heaviest tiles of a head all at once (a cohort that starts together and, each tile one unit
// shorter than the last, ends staggered); each freed slot takes the next-heaviest tile, so the
// following cohort starts staggered and ends together, and so on alternately.  Walking the keys
// upwards from key 0 in the cohorts that start together and downwards from the diagonal in those
// that end together keeps the workgroups of a cohort on about the same K/V tile at any moment, so
// one L2 fill of a tile serves all of them, where the staggered starts of a single direction
// spread them over the slots' worth of query tiles of K/V (4 MiB at d = 128 with 8192 query rows
// in flight: an L2's whole size).
__device__ __forceinline__ bool sched_descending(const Sched& s, int total) {
  if (!s.slots || !s.head_major) return false;
  int w = blockIdx.x;
  if (s.remap) w = (w & 7) * (total >> 3) + (w >> 3);
  const int r = w % (s.group * s.ntiles);  // position in the XCD's dispatch order
  return (r / s.slots) & 1;
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
