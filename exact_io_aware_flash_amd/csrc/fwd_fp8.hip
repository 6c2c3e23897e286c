// MX-FP8 forward pass for gfx950: E4M3 operands with power-of-two block scales on the scaled
// matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4), fp32 accumulation and softmax.
//
// Method: the same tiled forward with online softmax as the bf16 kernel ([P2] "FlashAttention:
// how a memory trick unlocked today's giant AI models", "Tiling: Breaking the Problem into
// Pieces" and "The Trick: Online Softmax"); FP8 arithmetic is the variant [P1] "How
// FlashAttention Bypasses the GPU Memory Bottleneck to Enable Long-Context AI" names for
// FlashAttention-3 (about 1.2 PFLOP/s on H100).  The pages fix no FP8 format; the one used is
// OCP MXFP8 (E4M3 elements, one E8M0 scale per 32 consecutive elements of the contraction
// index), the block-scaled format these matrix cores multiply natively.
//
// Inputs arrive quantised (the two quantisation kernels below, or any producer of the same
// layout): Q and K in blocks of 32 features, V transposed (feature-major) in blocks of 32 keys,
// so that both contractions (QK^T over features, PV over keys) see their block scales along
// the contraction index.  P is quantised in the kernel with scale 1 (P <= 2^8 < 448 under the
// lazy rescale below); the row sums use P in fp32, so LSE carries fp32 error only.
//
// Scaled MFMA operand layout (32 x 32 x 64, E4M3): lane l = 32 h + c holds row (A) or column
// (B) c; its byte j is contraction index k = 32 (j / 16) + 16 h + j % 16; its scale byte
// applies to row/column c and k-block h (k = 32 h .. 32 h + 31).  The output is the usual
// 32 x 32 fp32 layout (register r of lane l: row 8 (r / 4) + 4 h + r % 4, column c).
//
//  * S^T = K Q^T: A = K rows from LDS, B = Q (registers for the whole kernel).  A-row i loads
//    key pi(i) = 16 ((i >> 2) & 1) + 4 (i >> 3) + (i & 3) of its 32-key block, which puts key
//    16 h + r of the block in register r of lane half h: exactly the key of byte 16 kb + r of
//    the lane's P operand below.  So P^T = exp(S^T) feeds the PV MFMA from the lane's own
//    registers.
//  * O^T += V^T P^T: A = V^T rows (features) from LDS, B = P^T.
//  * K / V tiles of 64 keys arrive by asynchronous global->LDS copies, double-buffered, with a
//    16-byte-chunk XOR swizzle that keeps the 16-byte operand reads free of bank conflicts.
//  * Same software pipeline as the bf16 kernel: the exponentials of tile t run between the
//    score MFMAs of tile t+1; the row sums of tile t and the max of tile t+1 between the PV
//    MFMAs of tile t.
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kRescaleThresholdFp8 = 8.0f;  // log2 units: P <= 2^8 stays below E4M3's 448
constexpr float kE4M3Max = 448.f;
constexpr int kP8Scale = 127;  // E8M0 byte of 2^0: P is quantised unscaled

// ---------------------------------------------------------------------------------------------
// MX-FP8 quantisation of one block of 32 (OCP MX v1.0, section 6.3): shared exponent
// floor(log2(max |x|)) - 8 (8 = exponent of E4M3's largest normal), held to [-127, 127]; a
// zero block takes -127.  Elements x * 2^-e, clamped to +-448, rounded to nearest-even E4M3 by
// v_cvt_pk_fp8_f32 (which does not saturate by itself).  Inputs are finite.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int mx_exponent(float amax) {
  const int field = (int)((__float_as_uint(amax) >> 23) & 0xff);  // floor(log2) + 127 for normals
  return max(-127, min(127, field - 127 - 8));                     // zero / subnormal: -127
}

__device__ __forceinline__ float mx_scaled(float x, int e) {
  return fminf(fmaxf(__builtin_ldexpf(x, -e), -kE4M3Max), kE4M3Max);
}

// codes of four consecutive elements in one dword, first element in the low byte
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d, int e) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(a, e), mx_scaled(b, e), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(c, e), mx_scaled(d, e), r, true);
  return (uint32_t)r;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// One thread per block of 32 consecutive elements of x ([rows, d] bf16, d a multiple of 32).
__global__ __launch_bounds__(256) void mx_quantize_rows_kernel(const __bf16* __restrict__ x, uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales, long long nblocks) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = src[i];
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = bf16_lo(w4[j]);
      v[8 * i + 2 * j + 1] = bf16_hi(w4[j]);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_exponent(amax);
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = mx_pack4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], e);
  uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  scales[b] = (uint8_t)(e + 127);
}

// V [BH, N, D] bf16 -> V^T codes [BH, D, Np] and scales (blocks of 32 keys).  One workgroup per
// (head, 64-key chunk): the chunk is staged in LDS (rows >= N as zero), then thread (f, half)
// quantises the 32 keys 32 half .. 32 half + 31 of feature f.
template <int D>
__global__ __launch_bounds__(256) void mx_quantize_vt_kernel(const __bf16* __restrict__ v, uint8_t* __restrict__ codes_t,
                                                             uint8_t* __restrict__ scales_t, int N, int Np) {
  constexpr int ROWB = D * 2;  // bytes per staged row
  __shared__ __attribute__((aligned(16))) char tile[64 * ROWB];
  const int bh = blockIdx.y, k0 = blockIdx.x * 64, tid = threadIdx.x;
  const __bf16* head = v + (size_t)bh * N * D;
  constexpr int CHUNKS = 64 * ROWB / 16;
  for (int ch = tid; ch < CHUNKS; ch += 256) {
    const int row = ch / (ROWB / 16), col = ch % (ROWB / 16);
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (k0 + row < N) u = reinterpret_cast<const uint4*>(head + (size_t)(k0 + row) * D)[col];
    *reinterpret_cast<uint4*>(tile + row * ROWB + col * 16) = u;
  }
  __syncthreads();
  if (tid >= 2 * D) return;
  const int f = tid % D, half = tid / D;
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const unsigned short bits = *reinterpret_cast<const unsigned short*>(tile + (32 * half + i) * ROWB + 2 * f);
    x[i] = __uint_as_float((uint32_t)bits << 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const int e = mx_exponent(amax);
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = mx_pack4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3], e);
  uint4* dst = reinterpret_cast<uint4*>(codes_t + ((size_t)bh * D + f) * Np + k0 + 32 * half);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  const int kblk = k0 / 32 + half;
  scales_t[(((size_t)bh * (Np / 32) + kblk) * 32 + f % 32) * (D / 32) + f / 32] = (uint8_t)(e + 127);
}

// ---------------------------------------------------------------------------------------------
// Forward kernel
// ---------------------------------------------------------------------------------------------
// E4M3 x E4M3 with block scales: sa / sb hold the scale bytes of this lane's row / column, the
// byte used picked by OA / OB
template <int OA, int OB>
__device__ __forceinline__ f32x16 mfma_mx(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OA, sa, OB, sb);
}
// the same with both scale bytes chosen by a selector that is a constant after unrolling
__device__ __forceinline__ f32x16 mfma_mx_sel(int oa, int ob, i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  if (oa == 0 && ob == 0) return mfma_mx<0, 0>(a, b, c, sa, sb);
  if (oa == 1 && ob == 0) return mfma_mx<1, 0>(a, b, c, sa, sb);
  if (oa == 2 && ob == 0) return mfma_mx<2, 0>(a, b, c, sa, sb);
  if (oa == 3 && ob == 0) return mfma_mx<3, 0>(a, b, c, sa, sb);
  return mfma_mx<2, 2>(a, b, c, sa, sb);
}

template <int I>
using IC = std::integral_constant<int, I>;

// K tile: 64 key rows of D bytes; V^T tile: D feature rows of 64 bytes.  Chunk swizzles (16-byte
// chunks, 256-byte bank window): the 16 lanes of one read pass read one logical chunk of 16
// rows, so the (row mod rows-per-window, physical chunk) pairs must be distinct.  K rows in a
// pass are pi(0..15) or pi(16..31) (plus 32 kb): {0..7, 16..23} or {8..15, 24..31}.
template <int D>
__device__ __forceinline__ constexpr int sw_k8(int row) {
  return D >= 128 ? (((row >> 1) & 3) | (((row >> 4) & 1) << 2)) : (((row >> 2) & 1) | (((row >> 4) & 1) << 1));
}
__device__ __forceinline__ constexpr int sw_v8(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ constexpr int pi32(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

__device__ __forceinline__ i32x8 join16x2(uint4 a, uint4 b) {
  i32x8 r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}
__device__ __forceinline__ uint4 lds16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 2) void fwd_mxfp8_kernel(Fp8FwdArgs a, Sched sc) {
  constexpr int BR = 128, BC = 64;
  constexpr int DF = D / 64;   // 64-deep contraction chunks over d (score MFMAs per 32-key block)
  constexpr int DB = D / 32;   // 32-feature output blocks (PV MFMAs per tile)
  constexpr int NSB = D / 32;  // scale bytes per Q / K row
  constexpr int KT = BC * D, VT = D * BC;  // tile bytes
  constexpr int KCH = D / 16;              // 16-byte chunks per K row
  constexpr int KI = KT / 1024 / 4, VI = VT / 1024 / 4;  // copy instructions per wave and tile
  constexpr int NBUF = 4;
  // At d = 128 a tile's scales travel with its codes, copied into LDS (4 bytes per key of K,
  // 4 bytes per feature and 32-key block of V^T: 2 D bytes each, a quarter per wave, so that
  // every wave issues the same instructions); at d = 64 (2-byte K scale rows, which a 4-byte
  // copy could not range-check key by key) they are loaded into registers.
  constexpr bool LS = D == 128;
  constexpr int SB = 2 * D;  // scale bytes per tile (K and V^T alike)
  // vector-memory instructions per wave for one tile: the LDS copies and the scale copies/loads
  constexpr int KOPS = KI + (LS ? 1 : 2), VOPS = VI + 1;

  // four K and four V tile buffers: a tile's copy is issued three steps before its use.  Each
  // is an array of its own, so that the compiler can tell a read of one buffer from the copies
  // still in flight into the others (it would otherwise wait for every copy before each read).
  __shared__ __attribute__((aligned(1024))) char kbuf0[KT];
  __shared__ __attribute__((aligned(1024))) char kbuf1[KT];
  __shared__ __attribute__((aligned(1024))) char kbuf2[KT];
  __shared__ __attribute__((aligned(1024))) char kbuf3[KT];
  __shared__ __attribute__((aligned(1024))) char vbuf0[VT];
  __shared__ __attribute__((aligned(1024))) char vbuf1[VT];
  __shared__ __attribute__((aligned(1024))) char vbuf2[VT];
  __shared__ __attribute__((aligned(1024))) char vbuf3[VT];
  auto kbuf = [&](auto slot) -> char* {
    constexpr int r = decltype(slot)::value;
    if constexpr (r == 0) return kbuf0;
    else if constexpr (r == 1) return kbuf1;
    else if constexpr (r == 2) return kbuf2;
    else return kbuf3;
  };
  auto vbuf = [&](auto slot) -> char* {
    constexpr int r = decltype(slot)::value;
    if constexpr (r == 0) return vbuf0;
    else if constexpr (r == 1) return vbuf1;
    else if constexpr (r == 2) return vbuf2;
    else return vbuf3;
  };
  __shared__ __attribute__((aligned(16))) char ksb0[LS ? SB : 4];
  __shared__ __attribute__((aligned(16))) char ksb1[LS ? SB : 4];
  __shared__ __attribute__((aligned(16))) char ksb2[LS ? SB : 4];
  __shared__ __attribute__((aligned(16))) char ksb3[LS ? SB : 4];
  __shared__ __attribute__((aligned(16))) char vsb0[LS ? SB : 4];
  __shared__ __attribute__((aligned(16))) char vsb1[LS ? SB : 4];
  __shared__ __attribute__((aligned(16))) char vsb2[LS ? SB : 4];
  __shared__ __attribute__((aligned(16))) char vsb3[LS ? SB : 4];
  auto ksbuf = [&](auto slot) -> char* {
    constexpr int r = decltype(slot)::value;
    if constexpr (r == 0) return ksb0;
    else if constexpr (r == 1) return ksb1;
    else if constexpr (r == 2) return ksb2;
    else return ksb3;
  };
  auto vsbuf = [&](auto slot) -> char* {
    constexpr int r = decltype(slot)::value;
    if constexpr (r == 0) return vsb0;
    else if constexpr (r == 1) return vsb1;
    else if constexpr (r == 2) return vsb2;
    else return vsb3;
  };
  __shared__ unsigned short blist[SPARSE ? kMaxMaskBlocks : 1];
  __shared__ int bcount;

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5,
            c32 = lane & 31;
  const int N = a.N, Np = a.Np;
  int bh, qt;
  sched_decode(sc, gridDim.x, bh, qt);
  const int q0 = qt * BR;
  const uint8_t* __restrict__ K8 = a.k8 + (size_t)bh * N * D;
  const uint8_t* __restrict__ VT8 = a.vt8 + (size_t)bh * D * Np;

  // ---- key tiles this query block visits
  const int nk = (N + BC - 1) / BC;
  int ntiles = nk;
  if (CAUSAL) ntiles = min(ntiles, (min(q0 + BR, N) - 1) / BC + 1);
  if (SPARSE) {
    const int qb = q0 / kMaskBlock;
    const int hi = CAUSAL ? min(qb + 1, a.nb) : a.nb;
    if (w == 0) {
      const int cnt = build_block_list(a.mask, a.nb, qb, false, 0, hi, blist, lane);
      if (lane == 0) bcount = cnt;
    }
    __syncthreads();
    const int cnt = bcount;
    ntiles = 2 * cnt;
    if (cnt > 0 && (int)blist[cnt - 1] * kMaskBlock + BC >= N) ntiles -= 1;  // tail block half past N
  }
  // causal tiles of alternate cohorts walk the keys downwards from the diagonal (sched_descending);
  // the masks depend only on each tile's first key
  const bool desc = CAUSAL && !SPARSE && sched_descending(sc, gridDim.x);
  auto tile_start = [&](int t) -> int {
    if (SPARSE) return (int)blist[t >> 1] * kMaskBlock + (t & 1) * BC;
    return (desc ? ntiles - 1 - t : t) * BC;
  };

  // ---- Q operand (B): lane holds query q0 + 32 w + c32, features 64 f + 16 h .. and 64 f + 32 + 16 h ..
  const int qrow = q0 + 32 * w + c32;
  i32x8 qop[DF];
  int qsc = 0;
  {
    // rows past N load row N - 1 and are zeroed after: no branch around the loads, so they are
    // all in flight together
    const bool live = qrow < N;
    const size_t qr_row = (size_t)bh * N + min(qrow, N - 1);
    const uint8_t* qr = a.q8 + qr_row * D;
    const uint8_t* qs = a.qs + qr_row * NSB;
    const uint32_t srow = NSB == 4 ? *reinterpret_cast<const uint32_t*>(qs) : *reinterpret_cast<const unsigned short*>(qs);
    // a negative scale flips the sign bit of every Q code (exact), the exponent uses |scale|
    const uint32_t m = a.qsign;
#pragma unroll
    for (int f = 0; f < DF; ++f) {
      uint4 lo = *reinterpret_cast<const uint4*>(qr + 64 * f + 16 * h);
      uint4 hi4 = *reinterpret_cast<const uint4*>(qr + 64 * f + 32 + 16 * h);
      lo.x = live ? lo.x ^ m : 0u; lo.y = live ? lo.y ^ m : 0u; lo.z = live ? lo.z ^ m : 0u; lo.w = live ? lo.w ^ m : 0u;
      hi4.x = live ? hi4.x ^ m : 0u; hi4.y = live ? hi4.y ^ m : 0u;
      hi4.z = live ? hi4.z ^ m : 0u; hi4.w = live ? hi4.w ^ m : 0u;
      qop[f] = join16x2(lo, hi4);
    }
    qsc = live ? (int)(srow >> (8 * h)) : 0;  // byte 2f: block 2f + h
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = zero16();
  float m_used = neg_inf();  // running max in scaled log2 units
  float lsum = 0.f;
  const float sl = a.scale_log2;

  // ---- per-lane LDS read offsets
  int koff[2][DF][2];  // [kb][f][half]: K row 32 kb + pi(c32), chunks 4f + h and 4f + 2 + h
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int f = 0; f < DF; ++f)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = 32 * kb + pi32(c32), ch = 4 * f + 2 * u + h;
        koff[kb][f][u] = row * D + ((ch ^ sw_k8<D>(row)) << 4);
      }
  int voff[DB][2];  // V^T row 32 db + c32, chunks h and 2 + h
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = 32 * db + c32, ch = 2 * u + h;
      voff[db][u] = row * BC + ((ch ^ sw_v8(row)) << 4);
    }
  // ---- copy offsets: slot s = 64 (KI w + i) + lane of a tile
  int kcopy[KI], vcopy[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int s = 64 * (KI * w + i) + lane, row = s / KCH, pch = s % KCH;
    kcopy[i] = row * D + ((pch ^ sw_k8<D>(row)) << 4);
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int s = 64 * (VI * w + i) + lane, row = s / 4, pch = s % 4;
    vcopy[i] = row * Np + ((pch ^ sw_v8(row)) << 4);
  }
  auto issue_k = [&](char* buf, int k0) {
    lds_sentinel(buf + 1024 * KI * w, KI, lane);
    const Rsrc r = make_rsrc(K8 + (size_t)k0 * D, max(N - k0, 0) * D);
#pragma unroll
    for (int i = 0; i < KI; ++i) dma16(r, buf + 1024 * (KI * w + i), kcopy[i], 0);
  };
  auto issue_v = [&](char* buf, int k0) {
    lds_sentinel(buf + 1024 * VI * w, VI, lane);
    const Rsrc r = make_rsrc(VT8 + k0, D * Np - k0);
#pragma unroll
    for (int i = 0; i < VI; ++i) dma16(r, buf + 1024 * (VI * w + i), vcopy[i], 0);
  };
  // scale loads (registers): K rows of the two 32-key blocks, shifted so byte 2f is block 2f + h;
  // V^T: the DB bytes of feature 32 db + c32 (db = byte) in key block k0/32 + h
  const Rsrc ks_r = make_rsrc(a.ks + (size_t)bh * N * NSB, N * NSB);
  const Rsrc vs_r = make_rsrc(a.vts + (size_t)bh * (Np / 32) * 32 * DB, (Np / 32) * 32 * DB);
  auto load_ksc = [&](int k0, int (&out)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int off = (k0 + 32 * kb + pi32(c32)) * NSB;
      const uint32_t row = NSB == 4 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ks_r, off, 0, 0)
                                    : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(ks_r, off, 0, 0);
      out[kb] = (int)row;  // shifted by 8 h where used (a shift here would wait for the load)
    }
  };
  auto load_vsc = [&](int k0) -> int {
    const int off = ((k0 / 32 + h) * 32 + c32) * DB;
    return DB == 4 ? (int)__builtin_amdgcn_raw_buffer_load_b32(vs_r, off, 0, 0)
                   : (int)(uint32_t)__builtin_amdgcn_raw_buffer_load_b16(vs_r, off, 0, 0);
  };
  // LDS scale copy (d = 128): wave w copies bytes [SB/4 w, SB/4 (w + 1)) of the tile's scales,
  // starting at byte byte0 of the head's array, 4 bytes per lane (keys past N read as zero)
  auto copy_scales = [&](const Rsrc& r, char* dst, int byte0) {
    constexpr int PW = SB / 4;
#ifdef FA_CHECK
    if (lane < PW / 4) *reinterpret_cast<uint32_t*>(dst + PW * w + 4 * lane) = 0xFFFFFFFFu;  // NaN scale
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
    if (lane < PW / 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)(dst + PW * w), 4, byte0 + PW * w + 4 * lane, 0, 0, 0);
  };
  // the scales of a tile in slot r as the MFMAs take them: K rows of the two 32-key blocks
  // shifted so that byte 2f is block 2f + h; V^T: the DB bytes of feature 32 db + c32 (db = byte)
  // in key block h of the tile
  auto lds_ksc = [&](const char* src, int kb) -> int {
    return (int)(*reinterpret_cast<const uint32_t*>(src + (32 * kb + pi32(c32)) * 4) >> (8 * h));
  };
  auto lds_vsc = [&](const char* src) -> int { return *reinterpret_cast<const int*>(src + (32 * h + c32) * 4); };

  // S^T for the two 32-key blocks of a tile: register r of lane half h = key k0 + 32 kb + 16 h + r
  auto scores = [&](const char* tk, const int (&ksc)[2], f32x16(&s)[2]) {
    s[0] = zero16();
    s[1] = zero16();
#pragma unroll
    for (int f = 0; f < DF; ++f)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const i32x8 kop = join16x2(lds16(tk + koff[kb][f][0]), lds16(tk + koff[kb][f][1]));
        s[kb] = mfma_mx_sel(2 * f, 2 * f, kop, qop[f], s[kb], ksc[kb], qsc);
      }
  };
  auto mask_tile = [&](f32x16(&s)[2], int k0) {
    if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0 + 32 * w)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 16 * h + r;
          if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = neg_inf();
        }
    }
  };
  auto update_max = [&](const f32x16(&s)[2], float& m, float& alpha) {
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmax_nan(mt, s[kb][r]);
    mt = half_swap_max(mt) * sl;
    const float m_new = (mt > m + kRescaleThresholdFp8) ? mt : m;
    alpha = (m_new == m) ? 1.f : fast_exp2(m - m_new);
    m = m_new;
  };

  // Software pipeline: the scores one tile ahead of the exponentials, as in the bf16 kernel, but
  // the copies run further ahead, since a 64-key FP8 step holds half the matrix work of a bf16
  // one while a copy takes as long to land.  Tile i (its K and V copies and their scale loads)
  // lives in buffer slot i % 4.  Step t reads K[t+1] and V[t]; it issues K[t+4] and V[t+3] and
  // ends by waiting for K[t+2] and V[t+1] (issued in step t-2), so each copy has two steps to
  // land.  Vector-memory instructions complete in issue order, so that wait is a count: the
  // instructions of steps t-1 and t may stay in flight.
  f32x16 sbuf[2][2];
  int ksc[NBUF][2];
  int vsc[NBUF];
#pragma unroll
  for (int i = 0; i < NBUF; ++i) {
    ksc[i][0] = ksc[i][1] = kP8Scale;
    vsc[i] = kP8Scale;
  }
  auto issue_ktile = [&](int i, auto slot) {
    constexpr int r = decltype(slot)::value;
    const int k0 = tile_start(i);
    issue_k(kbuf(slot), k0);
    if constexpr (LS)
      copy_scales(ks_r, ksbuf(slot), k0 * NSB);
    else
      load_ksc(k0, ksc[r]);
  };
  auto issue_vtile = [&](int i, auto slot) {
    constexpr int r = decltype(slot)::value;
    const int k0 = tile_start(i);
    issue_v(vbuf(slot), k0);
    if constexpr (LS)
      copy_scales(vs_r, vsbuf(slot), k0 * DB);
    else
      vsc[r] = load_vsc(k0);
  };
  // scales of the tile in slot r, as the MFMAs take them
  auto kscales = [&](auto slot, int (&out)[2]) {
    constexpr int r = decltype(slot)::value;
    if constexpr (LS) {
      out[0] = lds_ksc(ksbuf(slot), 0);
      out[1] = lds_ksc(ksbuf(slot), 1);
    } else {
      out[0] = ksc[r][0] >> (8 * h);
      out[1] = ksc[r][1] >> (8 * h);
    }
  };
  auto vscale = [&](auto slot) -> int {
    constexpr int r = decltype(slot)::value;
    if constexpr (LS)
      return lds_vsc(vsbuf(slot));
    else
      return vsc[r];
  };
  float alpha = 1.f;
  if (ntiles > 0) issue_ktile(0, IC<0>{}), issue_vtile(0, IC<0>{});
  if (ntiles > 1) issue_ktile(1, IC<1>{}), issue_vtile(1, IC<1>{});
  if (ntiles > 2) issue_ktile(2, IC<2>{}), issue_vtile(2, IC<2>{});
  if (ntiles > 3) issue_ktile(3, IC<3>{});
  wait_dma();
  __syncthreads();
  if (ntiles > 0) {
    int ksc0[2];
    kscales(IC<0>{}, ksc0);
    scores(kbuf(IC<0>{}), ksc0, sbuf[0]);
    mask_tile(sbuf[0], tile_start(0));
    update_max(sbuf[0], m_used, alpha);
    alpha = 1.f;  // nothing accumulated yet
  }
  // every wave has read K[0] before step 0 copies K[4] over it
  if (ntiles > 4) lds_barrier();

  // P[t] as E4M3 codes, the PV operand (kept across steps: each word's first conversion keeps
  // the half it does not write)
  i32x8 pop = {0, 0, 0, 0, 0, 0, 0, 0};
  auto step = [&](int t, auto slot) {
    constexpr int r = decltype(slot)::value;  // t % 4
    constexpr int par = r & 1;                // t % 2
    // K[t+1] (stale K on the last tile: in bounds, result discarded) and its scales; V[t]
    const char* const k_next = kbuf(IC<(r + 1) % NBUF>{});
    int ksc_next[2];
    kscales(IC<(r + 1) % NBUF>{}, ksc_next);
    const char* const v_cur = vbuf(IC<r>{});
    const int vsc_cur = vscale(IC<r>{});
    f32x16(&s_cur)[2] = sbuf[par];
    f32x16(&s_nxt)[2] = sbuf[par ^ 1];
    const bool has1 = t + 1 < ntiles, has2 = t + 2 < ntiles, has3 = t + 3 < ntiles, has4 = t + 4 < ntiles;
    // K[t+4] into the slot of K[t] (read in step t-1), V[t+3] into that of V[t-1] (step t-1)
    if (has4) issue_ktile(t + 4, IC<r>{});
    if (has3) issue_vtile(t + 3, IC<(r + 3) % NBUF>{});

    if (wave_any(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
      lsum *= alpha;
    }
    const float msub = (m_used == neg_inf()) ? 0.f : m_used;

    // wave priority per section (two waves of different workgroups share a SIMD): the PV
    // section first, as measured
    __builtin_amdgcn_s_setprio(0);
    // section 1: S[t+1] on the matrix cores; P[t] = exp2(S[t] * scale * log2(e) - m) in fp32
    // (kept in s_cur for the row sums) and as E4M3 codes for PV: byte 16 kb + r of the operand
    // is register r of block kb.  Each MFMA is followed by a share of the exponentials.
    constexpr int NS = 2 * DF;
    constexpr int EPS = 32 / NS;
    // operands read two MFMAs ahead: K for this section, and V for the first two PV MFMAs of
    // section 2 in this section's last slots (an LDS read takes longer than one MFMA)
    auto kread = [&](int i) {
      const int f = i >> 1, kb = i & 1;
      return join16x2(lds16(k_next + koff[kb][f][0]), lds16(k_next + koff[kb][f][1]));
    };
    auto vread = [&](int db) { return join16x2(lds16(v_cur + voff[db][0]), lds16(v_cur + voff[db][1])); };
    i32x8 kop[NS], vop[DB];
    {
      s_nxt[0] = zero16();
      s_nxt[1] = zero16();
      kop[0] = kread(0);
      kop[1] = kread(1);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int f = i >> 1, kb = i & 1;
        if (i + 2 < NS)
          kop[i + 2] = kread(i + 2);
        else
          vop[i + 2 - NS] = vread(i + 2 - NS);  // V[t] landed before this step
        s_nxt[kb] = mfma_mx_sel(2 * f, 2 * f, kop[i], qop[f], s_nxt[kb], ksc_next[kb], qsc);
#pragma unroll
        for (int e = 0; e < EPS; ++e) {
          const int j = i * EPS + e;
          s_cur[j >> 4][j & 15] = fast_exp2(__builtin_fmaf(s_cur[j >> 4][j & 15], sl, -msub));
        }
#pragma unroll
        for (int e = 0; e < EPS; e += 4) {
          const int j = i * EPS + e;
          // the first conversion fills the low half of the word and keeps the rest of its old value
          // (the previous tile's, overwritten by the second one): no zeroing move
          int r = __builtin_amdgcn_cvt_pk_fp8_f32(s_cur[j >> 4][j & 15], s_cur[j >> 4][(j & 15) + 1], pop[j >> 2], false);
          r = __builtin_amdgcn_cvt_pk_fp8_f32(s_cur[j >> 4][(j & 15) + 2], s_cur[j >> 4][(j & 15) + 3], r, true);
          pop[j >> 2] = r;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // pin P[t] here: without a use in this section the compiler sinks the exponentials past the
    // mask branch below, away from the MFMAs they are meant to run beside
    asm volatile("" : "+v"(pop));
    asm volatile("" : "+v"(s_cur[0]), "+v"(s_cur[1]));
    __builtin_amdgcn_sched_barrier(0);

    if (has1) mask_tile(s_nxt, tile_start(t + 1));

    __builtin_amdgcn_s_setprio(1);
    // section 2: O^T += V^T P^T over the 64 keys, the row sums of P[t], the max after S[t+1].
    // Written out slot by slot like section 1: each PV MFMA is followed by its share of the row
    // sums and of the running max (V operands read two MFMAs ahead, the first two in section 1).
    {
      constexpr int EPD = 32 / DB;  // elements per slot
      float part[4] = {0.f, 0.f, 0.f, 0.f};
      float mt = s_nxt[0][0];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if (db + 2 < DB) vop[db + 2] = vread(db + 2);
        oacc[db] = mfma_mx_sel(db, 0, vop[db], pop, oacc[db], vsc_cur, kP8Scale);
#pragma unroll
        for (int e = 0; e < EPD; ++e) {
          const int j = db * EPD + e;
          part[j & 3] += s_cur[j >> 4][j & 15];
          mt = fmax_nan(mt, s_nxt[j >> 4][j & 15]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // keep the PV MFMAs, the sums and the max in this section: without uses here the compiler
      // sinks them past the select below, which it turns into a branch
#pragma unroll
      for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(oacc[db]));
      lsum += (part[0] + part[1]) + (part[2] + part[3]);
      asm volatile("" : "+v"(lsum));
      mt = half_swap_max(mt) * sl;
      float m_nx = (mt > m_used + kRescaleThresholdFp8) ? mt : m_used;
      float a_nx = (m_nx == m_used) ? 1.f : fast_exp2(m_used - m_nx);
      asm volatile("" : "+v"(m_nx), "+v"(a_nx));
      alpha = has1 ? a_nx : alpha;
      m_used = has1 ? m_nx : m_used;
    }
    __builtin_amdgcn_sched_barrier(0);
    // K[t+2] and V[t+1] have landed once at most the instructions of steps t-1 and t remain
    if (has4)
      wait_vm<2 * KOPS + 2 * VOPS>();
    else if (has3)
      wait_vm<KOPS + 2 * VOPS>();
    else if (has2)
      wait_vm<VOPS>();
    else
      wait_vm<0>();
    lds_barrier();
  };

  for (int t = 0; t < ntiles; t += 4) {
    step(t, IC<0>{});
    if (t + 1 < ntiles) step(t + 1, IC<1>{});
    if (t + 2 < ntiles) step(t + 2, IC<2>{});
    if (t + 3 < ntiles) step(t + 3, IC<3>{});
  }

  // ---- epilogue: lane holds features 32 db + 8 g + 4 h + e of query qrow in register 4 g + e
  const float ltot = half_swap_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (qrow < N) {
    __bf16* orow = a.o + ((size_t)bh * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(oacc[db][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g + 4 * h) = v4;
      }
    if (h == 0) a.lse[(size_t)bh * N + qrow] = ltot > 0.f ? (m_used + __log2f(ltot)) * kLn2 : neg_inf();
  }
}

}  // namespace

template <int D, bool C, bool S>
static hipError_t launch_fp8_t(const Fp8FwdArgs& a, hipStream_t st) {
  constexpr int BR = 128;
  const int nq = (a.N + BR - 1) / BR;
  static const int slots = xcd_slots(reinterpret_cast<const void*>(&fwd_mxfp8_kernel<D, C, S>));
  const Sched sc = make_sched(nq, a.BH, /*heavy_last_tile=*/1, slots, /*uneven=*/C || S, /*alternate=*/C && !S);
  hipLaunchKernelGGL((fwd_mxfp8_kernel<D, C, S>), dim3(nq * a.BH), dim3(256), 0, st, a, sc);
  return hipGetLastError();
}

hipError_t launch_fwd_mxfp8(const Fp8FwdArgs& a, hipStream_t stream) {
  const bool causal = a.causal != 0, sparse = a.mask != nullptr;
  if (a.d == 64) {
    if (causal) return sparse ? launch_fp8_t<64, true, true>(a, stream) : launch_fp8_t<64, true, false>(a, stream);
    return sparse ? launch_fp8_t<64, false, true>(a, stream) : launch_fp8_t<64, false, false>(a, stream);
  }
  if (causal) return sparse ? launch_fp8_t<128, true, true>(a, stream) : launch_fp8_t<128, true, false>(a, stream);
  return sparse ? launch_fp8_t<128, false, true>(a, stream) : launch_fp8_t<128, false, false>(a, stream);
}

hipError_t launch_mxfp8_quantize_rows(const __bf16* x, uint8_t* codes, uint8_t* scales, long long rows, int d,
                                      hipStream_t st) {
  const long long nblocks = rows * (d / 32);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quantize_rows_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, st, x, codes,
                     scales, nblocks);
  return hipGetLastError();
}

hipError_t launch_mxfp8_quantize_vt(const __bf16* v, uint8_t* codes_t, uint8_t* scales_t, int BH, int N, int d,
                                    hipStream_t st) {
  const int Np = fp8_vt_cols(N);
  const dim3 grid(Np / 64, BH);
  if (d == 64)
    hipLaunchKernelGGL((mx_quantize_vt_kernel<64>), grid, dim3(256), 0, st, v, codes_t, scales_t, N, Np);
  else
    hipLaunchKernelGGL((mx_quantize_vt_kernel<128>), grid, dim3(256), 0, st, v, codes_t, scales_t, N, Np);
  return hipGetLastError();
}

}  // namespace fa
