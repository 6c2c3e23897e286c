// Forward pass, bf16 inputs, fp32 accumulation, for gfx950.
//
// Method ([P2] "FlashAttention: how a memory trick unlocked today's giant AI models",
// sections "Tiling: Breaking the Problem into Pieces" and "The Trick: Online Softmax"): each
// workgroup owns a block of query rows, walks the key/value tiles, and keeps per row a running
// maximum and a running sum of exponentials; S and P for a tile live only in registers.  The
// output block is divided by the sum once at the end and the row statistic
// LSE = max + ln(sum) is stored for the backward pass ([P3] "How FlashAttention Eliminates
// Transformer Memory Bottlenecks", "Innovation #3").  Masked 128 x 128 blocks are skipped
// ([P3] "Innovation #5").
//
// gfx950 mapping
//  * workgroup = 4 waves x 32 query rows (BR = 128 rows, one mask block), K/V tiles of BC = 64
//    keys double-buffered in LDS (global loads for tile t+1 are issued before the math of tile t
//    and written to the other buffer after it; one barrier per tile).
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: Q^T is the B operand, held in registers for the
//    whole kernel; K rows are the A operand (16-byte LDS reads).  Each lane then holds one query
//    (lane % 32) and 16 keys per 32-key block, so the row max and row sum are in-lane plus one
//    v_permlane32_swap between the two wave halves.
//  * O^T += V^T P^T: P^T (bf16, from the S^T registers) is the B operand as is; V^T is read
//    transposed from the row-major V tile with ds_read_b64_tr_b16.
//  * exponentials in base 2 with scale*log2(e) folded into one FMA; the running maximum is only
//    moved when a new score exceeds it by more than 2^8, so most tiles skip the O rescale (the
//    result is the same: numerator and denominator always share the offset).
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a, Sched sc) {
  constexpr int BR = 128, BC = 64;
  constexpr int DC = D / 16;                // 16-wide contraction chunks over d
  constexpr int DB = D / 32;                // 32-row output blocks over d
  constexpr int TILE_BYTES = BC * D * 2;
  constexpr int CH = TILE_BYTES / 16 / 256;  // 16-byte chunks per thread per tile
  constexpr int CPR = D / 8;                 // 16-byte chunks per row

  __shared__ __attribute__((aligned(16))) char lds_k[2][TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_v[2][TILE_BYTES];
  __shared__ unsigned short blist[SPARSE ? kMaxMaskBlocks : 1];
  __shared__ int bcount;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, c32 = lane & 31;
  const int N = a.N;
  int bh, qt;
  sched_decode(sc, gridDim.x, bh, qt);
  const int q0 = qt * BR;
  const size_t base = (size_t)bh * N * D;
  const __bf16* __restrict__ Q = a.q + base;
  const __bf16* __restrict__ K = a.k + base;
  const __bf16* __restrict__ V = a.v + base;

  // ---- key tiles this query block visits
  const int nk = (N + BC - 1) / BC;
  int kv_end = nk;
  if (CAUSAL) kv_end = min(nk, (min(q0 + BR, N) - 1) / BC + 1);
  int ntiles = kv_end;
  if (SPARSE) {
    const int qb = q0 / kMaskBlock;
    const int hi = CAUSAL ? qb + 1 : a.nb;
    if (w == 0) {
      const int cnt = build_block_list(a.mask, a.nb, qb, false, 0, hi, blist, lane);
      if (lane == 0) bcount = cnt;
    }
    __syncthreads();
    const int cnt = bcount;
    ntiles = 2 * cnt;
    if (cnt > 0 && (int)blist[cnt - 1] * kMaskBlock + BC >= N) ntiles -= 1;  // tail block half past N
  }
  auto tile_start = [&](int t) -> int {
    if (SPARSE) return (int)blist[t >> 1] * kMaskBlock + (t & 1) * BC;
    return t * BC;
  };

  // ---- Q^T operand in registers
  const int qrow = q0 + 32 * w + c32;
  bf16x8 qreg[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c)
    qreg[c] = qrow < N ? *reinterpret_cast<const bf16x8*>(Q + (size_t)qrow * D + 16 * c + 8 * h) : zero_bf16x8();

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = zero16();
  float m_used = neg_inf();  // running max in scaled log2 units
  float lsum = 0.f;          // this lane's partial sum of exponentials
  const float sl = a.scale_log2;

  // ---- global -> registers -> LDS staging of one K/V tile
  uint4 kpre[CH], vpre[CH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / CPR, col = (cidx % CPR) * 8;
      const int key = k0 + row;
      if (key < N) {
        kpre[i] = *reinterpret_cast<const uint4*>(K + (size_t)key * D + col);
        vpre[i] = *reinterpret_cast<const uint4*>(V + (size_t)key * D + col);
      } else {
        kpre[i] = make_uint4(0, 0, 0, 0);
        vpre[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int cidx = tid + 256 * i;
      const int row = cidx / CPR, col = (cidx % CPR) * 8;
      *reinterpret_cast<uint4*>(lds_k[buf] + lds_off<D>(row, col)) = kpre[i];
      *reinterpret_cast<uint4*>(lds_v[buf] + lds_off<D>(row, col)) = vpre[i];
    }
  };

  if (ntiles > 0) {
    gload(tile_start(0));
    lstore(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int k0 = tile_start(t);
    const bool has_next = t + 1 < ntiles;
    if (has_next) gload(tile_start(t + 1));
    const char* tk = lds_k[buf];
    const char* tv = lds_v[buf];

    // S^T = K Q^T for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int c = 0; c < DC; ++c) s[kb] = mfma32(lds_row8<D>(tk, kb * 32 + c32, 16 * c + 8 * h), qreg[c], s[kb]);
    }

    // element masks: the causal diagonal and the key tail
    const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0 + 32 * w);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = neg_inf();
        }
    }

    // online softmax
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = half_swap_max(mt) * sl;
    const float m_new = (mt > m_used + kRescaleThreshold) ? mt : m_used;
    const float alpha = (m_new == m_used) ? 1.f : fast_exp2(m_used - m_new);
    m_used = m_new;
    if (wave_any(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
      lsum *= alpha;
    }
    const float msub = (m_used == neg_inf()) ? 0.f : m_used;

    // P in fp32 feeds the row sum (so LSE carries fp32 error only); its bf16 rounding feeds PV
    bf16x8 pk[4];
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = fast_exp2(__builtin_fmaf(s[kb][8 * u + e], sl, -msub));
          part[e & 3] += pv;
          pk[2 * kb + u][e] = (__bf16)pv;
        }
    lsum += (part[0] + part[1]) + (part[2] + part[3]);

    // O^T += V^T P^T over the 64 keys (4 contraction chunks of 16)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) oacc[db] = mfma32(lds_tr_operand<D>(tv, 16 * m, 32 * db, lane), pk[m], oacc[db]);

    if (has_next) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const float ltot = half_swap_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (qrow < N) {
    __bf16* orow = a.o + base + (size_t)qrow * D;
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
static hipError_t launch_fwd_t(const FwdArgs& a, const Sched& sc, int grid, hipStream_t st) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, C, S>), dim3(grid), dim3(256), 0, st, a, sc);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  constexpr int BR = 128;
  const int nq = (a.N + BR - 1) / BR;
  const Sched sc = make_sched(nq, a.BH, /*heavy_last_tile=*/1);
  const int grid = nq * a.BH;
  const bool causal = a.causal != 0, sparse = a.mask != nullptr;
  if (a.d == 64) {
    if (causal) return sparse ? launch_fwd_t<64, true, true>(a, sc, grid, stream) : launch_fwd_t<64, true, false>(a, sc, grid, stream);
    return sparse ? launch_fwd_t<64, false, true>(a, sc, grid, stream) : launch_fwd_t<64, false, false>(a, sc, grid, stream);
  }
  if (causal) return sparse ? launch_fwd_t<128, true, true>(a, sc, grid, stream) : launch_fwd_t<128, true, false>(a, sc, grid, stream);
  return sparse ? launch_fwd_t<128, false, true>(a, sc, grid, stream) : launch_fwd_t<128, false, false>(a, sc, grid, stream);
}

}  // namespace fa
