// Library-internal argument blocks and launchers (host side).  Arguments have already been
// validated by the C ABI layer (api.cpp) when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_common.h"

namespace fa {

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  const uint8_t* mask;  // nullptr = dense
  int N, d, BH, nb, causal;
  float scale;       // natural-units scale (either sign)
  float scale_log2;  // |scale| * log2(e)
  // sign of scale folded into the Q operand: 0x80008000 flips both bf16 of a dword (exact), 0
  // leaves them; S = |scale| (sign * Q) K^T is then the scaled score for either sign
  uint32_t qsign;
  // split-key forward: the 128-key blocks are cut into `splits` contiguous ranges (range s =
  // blocks [s * nb / splits, (s + 1) * nb / splits)); range s writes its normalised partial
  // output to o_part[s] (float32 [BH, N, d]) and its log-sum-exp to lse_part[s] ([BH, N])
  int splits;
  float* o_part;
  float* lse_part;
};

// Split-key forward workspace: float32 partial outputs [splits, BH, N, d] followed by partial
// log-sum-exps [splits, BH, N], each part 256-byte aligned.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t splitkv_o_bytes(long long BH, int N, int d, int splits) { return align256((size_t)splits * BH * N * d * 4); }
inline size_t splitkv_ws_bytes(long long BH, int N, int d, int splits) {
  return splitkv_o_bytes(BH, N, d, splits) + align256((size_t)splits * BH * N * 4);
}

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* delta;  // workspace: D = rowsum(dO * O), [BH, N]
  const uint8_t* mask;
  int N, d, BH, nb, causal;
  float scale;       // signed: multiplies dK and dQ at the end
  float scale_log2;  // |scale| * log2(e)
  // sign of scale folded into the operand held in registers for S (Q in the dQ kernel, K in the
  // dK/dV kernels): 0x80008000 per dword of bf16 pairs, or 0
  uint32_t ssign;
};

// Backward workspace: delta (float32 [BH, N]), 256-byte aligned size.
inline size_t ws_bytes(long long BH, int N) { return ((size_t)BH * N * 4 + 255) & ~(size_t)255; }

// Fixed device scratch of the allocation-free backward: float32 D for at most 2^22 query rows
// (B * H * N), 16 MiB per device.  noalloc_scratch() returns the current device's address of the
// array (looked up once per device); it allocates nothing.
constexpr long long kNoallocMaxRows = 1LL << 22;
constexpr size_t kNoallocScratchBytes = (size_t)kNoallocMaxRows * 4;
hipError_t noalloc_scratch(void** out);

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  const float* dout;
  float* out_o;
  float* lse;  // written by the forward, read by the backward
  float* dq;
  float* dk;
  float* dv;
  float* delta;
  const uint8_t* mask;
  int N, d, BH, nb, causal;
  float scale;
};

// Workgroups of `kernel` (block_threads threads each) resident at once on one XCD: occupancy
// per CU times the CUs of one of the 8 XCDs.  Asked once per kernel instantiation (the caller
// caches it).
inline int xcd_slots(const void* kernel, int block_threads = 256) {
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    cus = 256;
  (void)hipGetLastError();  // a failed query must not surface as the launch's error
  return per_cu * (cus / 8);
}

// `uneven`: the tiles of a head differ in work (causal triangle, block mask).  Tiles of equal
// work always run head-major (no imbalance to fear, and the workgroups in flight share a head's
// stream in L2: 11-20% on non-causal heads of N = 2048..8192 at d = 128); uneven ones once a head
// has at least as many tiles as the XCD has resident workgroups, below which the long tiles of
// the last heads would start too late (25% slower on causal d = 64 heads of N = 2048).
inline Sched make_sched(int ntiles, int BH, int heavy_last_tile, int slots_per_xcd, bool uneven, bool alternate = false) {
  Sched s;
  s.ntiles = ntiles;
  s.heavy_last_tile = heavy_last_tile;
  s.slots = alternate ? slots_per_xcd : 0;
  if (BH % 8 == 0) {
    s.remap = 1;
    s.group = BH / 8;
    s.head_major = uneven ? ntiles >= slots_per_xcd : 1;
  } else {
    s.remap = 0;
    s.group = BH;
    s.head_major = 0;
  }
  return s;
}

// MX-FP8 forward: E4M3 element codes with one E8M0 scale per block of 32.  Q and K are
// row-quantised ([BH, N, d] codes, [BH, N, d/32] scales, blocks along d); V is stored transposed
// ([BH, d, Np] codes, keys >= N zero, Np = N rounded up to 64) with blocks of 32 keys, scale of
// (feature f, key block j) at ((bh * Np/32 + j) * 32 + f % 32) * (d/32) + f / 32.
struct Fp8FwdArgs {
  const uint8_t* q8;
  const uint8_t* qs;
  const uint8_t* k8;
  const uint8_t* ks;
  const uint8_t* vt8;
  const uint8_t* vts;
  __bf16* o;
  float* lse;
  const uint8_t* mask;
  int N, Np, d, BH, nb, causal;
  float scale_log2;  // |scale| * log2(e)
  uint32_t qsign;    // 0x80808080 flips the sign bit of four E4M3 Q codes (scale < 0), or 0
};
inline int fp8_vt_cols(int N) { return (N + 63) / 64 * 64; }

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
// the wave-specialised forward (d = 128, no block mask, no split)
hipError_t launch_fwd_pingpong_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_mxfp8(const Fp8FwdArgs& a, hipStream_t stream);
// MX-FP8 quantisation of bf16 rows (blocks of 32 along d), and of V into the transposed layout
hipError_t launch_mxfp8_quantize_rows(const __bf16* x, uint8_t* codes, uint8_t* scales, long long rows, int d,
                                      hipStream_t stream);
hipError_t launch_mxfp8_quantize_vt(const __bf16* v, uint8_t* codes_t, uint8_t* scales_t, int BH, int N, int d,
                                    hipStream_t stream);
// split-key forward: partials into a.o_part / a.lse_part, then the log-sum-exp merge into a.o / a.lse
hipError_t launch_fwd_splitkv_bf16(const FwdArgs& a, hipStream_t stream);
// log-sum-exp merge of `parts` partial results over disjoint key sets of the same `rows` rows
hipError_t launch_merge_bf16(const float* o_parts, const float* lse_parts, int parts, long long rows, int d,
                             __bf16* o, float* lse, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_delta_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const BwdArgs& a, hipStream_t stream);
// one-pass backward (d = 128): the pre-pass also zeroes the float32 dQ accumulator [BH, N, d],
// one kernel computes dK, dV and adds dQ with atomics, a last one converts dQ to bf16 (x scale)
inline size_t dq_acc_bytes(long long BH, int N, int d) { return (size_t)BH * N * d * 4; }
hipError_t launch_bwd_onepass_bf16(const BwdArgs& a, float* dq_acc, hipStream_t stream);
hipError_t launch_bwd_prepass_zero_bf16(const BwdArgs& a, float* dq_acc, hipStream_t stream);
hipError_t launch_bwd_dkdvq_bf16(const BwdArgs& a, float* dq_acc, hipStream_t stream);
hipError_t launch_bwd_dq_convert_bf16(const BwdArgs& a, const float* dq_acc, hipStream_t stream);
hipError_t launch_fwd_f32(const F32Args& a, hipStream_t stream);
hipError_t launch_bwd_f32(const F32Args& a, hipStream_t stream);

}  // namespace fa
