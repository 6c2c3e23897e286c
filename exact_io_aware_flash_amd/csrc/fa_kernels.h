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
  float scale;       // natural-units scale
  float scale_log2;  // scale * log2(e)
};

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
  float scale, scale_log2;
};

// Backward workspace: delta (float32 [BH, N]), 256-byte aligned size.
inline size_t ws_bytes(long long BH, int N) { return ((size_t)BH * N * 4 + 255) & ~(size_t)255; }

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

inline Sched make_sched(int ntiles, int BH, int heavy_last_tile, int slots_per_xcd) {
  Sched s;
  s.ntiles = ntiles;
  s.heavy_last_tile = heavy_last_tile;
  if (BH % 8 == 0) {
    s.remap = 1;
    s.group = BH / 8;
    s.head_major = ntiles >= 2 * slots_per_xcd;
  } else {
    s.remap = 0;
    s.group = BH;
    s.head_major = 0;
  }
  return s;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_delta_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const F32Args& a, hipStream_t stream);
hipError_t launch_bwd_f32(const F32Args& a, hipStream_t stream);

}  // namespace fa
