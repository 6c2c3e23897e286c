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
//    keys copied global -> LDS asynchronously (buffer_load ... lds: no registers, no VALU) and
//    software-pipelined: while the exponentials of tile t run on the VALU, the MFMAs already
//    compute the scores of tile t+1, so K is copied two tiles ahead and V one tile ahead (each
//    double-buffered; one barrier per tile).
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: Q^T is the B operand, held in registers for the
//    whole kernel; K rows are the A operand (16-byte LDS reads).  Each lane then holds one query
//    (lane % 32) and 16 keys per 32-key block, so the row max and row sum are in-lane plus one
//    v_permlane32_swap between the two wave halves.
//  * O^T += V^T P^T: P^T (bf16, from the S^T registers) is the B operand as is; V^T is read
//    from the row-major V tile with the transposing ds_read_b64_tr_b16.  K rows are read in a
//    bit-permuted order that makes each lane's 8 P values 8 consecutive keys.  Both tiles use
//    a 16-byte-chunk XOR swizzle that keeps their reads free of LDS bank conflicts.
//  * exponentials in base 2 with scale*log2(e) folded into one FMA; the running maximum is only
//    moved when a new score exceeds it by more than 2^8, so most tiles skip the O rescale (the
//    result is the same: numerator and denominator always share the offset).
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <int D, bool CAUSAL, bool SPARSE, bool SPLIT = false>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a, Sched sc) {
  constexpr int BR = 128, BC = 64;
  constexpr int DC = D / 16;  // 16-wide contraction chunks over d
  constexpr int DB = D / 32;  // 32-row output blocks over d
  using KT = DmaTile<BC, D>;  // K rows, read 16 bytes per lane
  using VT = DmaTile<BC, D>;  // V rows, read transposed (ds_read_b64_tr_b16)

  __shared__ __attribute__((aligned(1024))) char kbuf0[KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf1[KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[VT::BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf1[VT::BYTES];
  __shared__ unsigned short blist[SPARSE ? kMaxMaskBlocks : 1];
  __shared__ int bcount;

  // the wave index is uniform: held in a scalar register, the LDS targets of the copies need no
  // per-issue v_readfirstlane
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5,
            c32 = lane & 31;
  const int N = a.N;
  int bh, qt;
  sched_decode(sc, gridDim.x, bh, qt);
  const int q0 = qt * BR;
  const size_t base = (size_t)bh * N * D;
  const __bf16* __restrict__ Q = a.q + base;
  const __bf16* __restrict__ K = a.k + base;
  const __bf16* __restrict__ V = a.v + base;

  // ---- key tiles this query block visits: all of them, or (split-key forward) those of the
  // 128-key blocks [blo, bhi) of range blockIdx.y
  const int nk = (N + BC - 1) / BC;
  const int blo = SPLIT ? (int)((long long)blockIdx.y * a.nb / a.splits) : 0;
  const int bhi = SPLIT ? (int)((long long)(blockIdx.y + 1) * a.nb / a.splits) : a.nb;
  const int tlo = 2 * blo;
  int tend = SPLIT ? min(nk, 2 * bhi) : nk;  // one past the last tile
  if (CAUSAL) tend = min(tend, (min(q0 + BR, N) - 1) / BC + 1);
  int ntiles = max(tend - tlo, 0);
  if (SPARSE) {
    const int qb = q0 / kMaskBlock;
    const int hi = CAUSAL ? min(qb + 1, bhi) : bhi;
    if (w == 0) {
      const int cnt = build_block_list(a.mask, a.nb, qb, false, blo, hi, blist, lane);
      if (lane == 0) bcount = cnt;
    }
    __syncthreads();
    const int cnt = bcount;
    ntiles = 2 * cnt;
    if (cnt > 0 && (int)blist[cnt - 1] * kMaskBlock + BC >= N) ntiles -= 1;  // tail block half past N
  }
  auto tile_start = [&](int t) -> int {
    if (SPARSE) return (int)blist[t >> 1] * kMaskBlock + (t & 1) * BC;
    return (tlo + t) * BC;
  };

  // ---- Q^T operand in registers (B operand: lane holds query q0 + 32w + c32, features 16c + 8h ..)
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

  // ---- per-lane LDS addresses (the chunk swizzle of each tile depends only on the lane)
  // K operand: row 32 kb + perm32(c32), features 16c + 8h .. (one 16-byte chunk)
  int kaddr[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) kaddr[c] = KT::off(perm32(c32), 16 * c + 8 * h);
  // V^T operand, transposed read u (u = 0, 1) of feature block db: lane j of its 16-lane group
  // addresses key row 16m + 8h + 4u + j/4 (16m added per use), features 32db + 16g + 4(j%4) ..
  int vaddr[2][DB];
  {
    const int g = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 8 * h + 4 * u + (j >> 2), col = 32 * db + 16 * g + 4 * (j & 3);
        vaddr[u][db] = VT::off4(row, col);
      }
  }

  KT kdma;
  VT vdma;
  kdma.init(w, lane);
  vdma.init(w, lane);

  // S^T = K Q^T for two 32-key blocks; register r of half h holds key k0 + 32 kb + acc_row(r, h)
  // the two 32-key blocks alternate, so consecutive MFMAs are independent; K reads run four
  // MFMAs ahead of their use (the scheduling groups keep the compiler from sinking them)
  auto scores = [&](const char* tk, f32x16(&s)[2]) {
    s[0] = zero16();
    s[1] = zero16();
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(lds_b128(tk + kaddr[c] + 32 * kb * D * 2), qreg[c], s[kb]);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * DC - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };

  // Software pipeline over key tiles (K runs one tile ahead of V):
  //   iteration t:  copies of K[t+2], V[t+1] in flight;  softmax of S[t] next to the MFMAs of
  //                 S[t+1] = K[t+1] Q^T;  O += V[t] P[t];  wait for the copies; barrier.
  // K tiles alternate between kbuf0/kbuf1 and V tiles between vbuf0/vbuf1, so the buffer a copy
  // lands in during iteration t is never one read in iteration t.  The scores alternate between
  // sbuf[0] and sbuf[1] the same way, so no step copies registers.
  f32x16 sbuf[2][2];
  if (ntiles > 0) {
    kdma.issue(K, N, kbuf0, tile_start(0), w);
    vdma.issue(V, N, vbuf0, tile_start(0), w);
    if (ntiles > 1) kdma.issue(K, N, kbuf1, tile_start(1), w);
  }
  wait_dma();
  __syncthreads();
  if (ntiles > 0) scores(kbuf0, sbuf[0]);

  auto step = [&](int t, auto parity) {
    constexpr int par = decltype(parity)::value;  // t % 2
    char* const k_next = par ? kbuf0 : kbuf1;      // holds K[t+1]
    char* const k_free = par ? kbuf1 : kbuf0;      // held K[t]; receives K[t+2]
    char* const v_cur = par ? vbuf1 : vbuf0;       // holds V[t]
    char* const v_free = par ? vbuf0 : vbuf1;      // held V[t-1]; receives V[t+1]
    f32x16(&s_cur)[2] = sbuf[par];
    f32x16(&s_nxt)[2] = sbuf[par ^ 1];
    const int k0 = tile_start(t);
    const bool has1 = t + 1 < ntiles, has2 = t + 2 < ntiles;
    if (has2) kdma.issue(K, N, k_free, tile_start(t + 2), w);
    if (has1) vdma.issue(V, N, v_free, tile_start(t + 1), w);

    // element masks: the causal diagonal and the key tail
    const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0 + 32 * w);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + acc_row(r, h);
          if (key >= N || (CAUSAL && key > qrow)) s_cur[kb][r] = neg_inf();
        }
    }

    // online softmax: running max moves only when a score exceeds it by more than 2^8
    float mt = s_cur[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmax_nan(mt, s_cur[kb][r]);
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

    // next tile's scores: independent of the exponentials below, so the two can overlap.
    // MFMA sections run at raised wave priority, so that when both waves of a SIMD can issue,
    // the one feeding the matrix pipe goes first and the other's softmax fills the gaps
    __builtin_amdgcn_s_setprio(1);
    if (has1) scores(k_next, s_nxt);
    __builtin_amdgcn_s_setprio(0);

    // P in fp32 feeds the row sum (so LSE carries fp32 error only); its bf16 rounding feeds PV.
    // pk[2 kb + m2] holds keys k0 + 32 kb + 16 m2 + 8h + 0..7: one k-slot group of the PV MFMA.
    bf16x8 pk[4];
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = fast_exp2(__builtin_fmaf(s_cur[kb][8 * m2 + e], sl, -msub));
          part[e & 3] += pv;
          pk[2 * kb + m2][e] = (__bf16)pv;
        }
    lsum += (part[0] + part[1]) + (part[2] + part[3]);

    __builtin_amdgcn_s_setprio(1);
    // O^T += V^T P^T over the 64 keys (4 contraction chunks of 16; V^T read transposed)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const char* vb = v_cur + 16 * m * D * 2;
        oacc[db] = mfma32(join8(lds_tr4(vb + vaddr[0][db]), lds_tr4(vb + vaddr[1][db])), pk[m], oacc[db]);
      }
    // each PV MFMA takes one transposed operand (two 8-byte reads), kept two MFMAs ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int i = 0; i < 4 * DB - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);

    __builtin_amdgcn_s_setprio(0);
    wait_dma();
    __syncthreads();
  };

  for (int t = 0; t < ntiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: lane holds features 32 db + 8 g + 4 h + e of query qrow in register 4 g + e
  const float ltot = half_swap_sum(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (SPLIT) {
    if (qrow < N) {
      const size_t prow = ((size_t)blockIdx.y * a.BH + bh) * N + qrow;
      float* orow = a.o_part + prow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = oacc[db][4 * g + e] * inv;
          *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * h) = v4;
        }
      if (h == 0) a.lse_part[prow] = ltot > 0.f ? (m_used + __log2f(ltot)) * kLn2 : neg_inf();
    }
    return;
  }
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


// ---------------------------------------------------------------------------------------------
// Log-sum-exp merge of partial results over disjoint key sets of the same query rows: with
// LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s, which is the softmax over the union
// of the key sets (each O_s is already normalised by its own sum).  Rows whose parts are all
// dead (LSE_s = -inf) get O = 0 and LSE = -inf.  TPR threads per row, 4 features per thread.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_parts, const float* __restrict__ lse_parts,
                                                    int parts, long long rows, __bf16* __restrict__ o,
                                                    float* __restrict__ lse) {
  constexpr int TPR = D / 4, RPB = 256 / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int f = 4 * (threadIdx.x % TPR);
  if (row >= rows) return;
  float m = neg_inf();
  for (int s = 0; s < parts; ++s) m = fmaxf(m, lse_parts[(size_t)s * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != neg_inf()) {
    for (int s = 0; s < parts; ++s) {
      const float ls = lse_parts[(size_t)s * rows + row];
      const float wt = fast_exp2((ls - m) * kLog2e);  // 0 for a dead part
      wsum += wt;
      const f32x4 v = *reinterpret_cast<const f32x4*>(o_parts + ((size_t)s * rows + row) * D + f);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(wt, v[e], acc[e]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  bf16x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = (__bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x4*>(o + (size_t)row * D + f) = out;
  if (f == 0) lse[row] = wsum > 0.f ? m + __logf(wsum) : neg_inf();
}

}  // namespace

template <int D, bool C, bool S>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  constexpr int BR = 128;
  const int nq = (a.N + BR - 1) / BR;
  static const int slots = xcd_slots(reinterpret_cast<const void*>(&fwd_bf16_kernel<D, C, S>));
  const Sched sc = make_sched(nq, a.BH, /*heavy_last_tile=*/1, slots);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, C, S>), dim3(nq * a.BH), dim3(256), 0, st, a, sc);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  const bool causal = a.causal != 0, sparse = a.mask != nullptr;
  if (a.d == 64) {
    if (causal) return sparse ? launch_fwd_t<64, true, true>(a, stream) : launch_fwd_t<64, true, false>(a, stream);
    return sparse ? launch_fwd_t<64, false, true>(a, stream) : launch_fwd_t<64, false, false>(a, stream);
  }
  if (causal) return sparse ? launch_fwd_t<128, true, true>(a, stream) : launch_fwd_t<128, true, false>(a, stream);
  return sparse ? launch_fwd_t<128, false, true>(a, stream) : launch_fwd_t<128, false, false>(a, stream);
}

template <int D, bool C, bool S>
static hipError_t launch_splitkv_t(const FwdArgs& a, hipStream_t st) {
  constexpr int BR = 128;
  const int nq = (a.N + BR - 1) / BR;
  static const int slots = xcd_slots(reinterpret_cast<const void*>(&fwd_bf16_kernel<D, C, S, true>));
  const Sched sc = make_sched(nq, a.BH, /*heavy_last_tile=*/1, slots);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, C, S, true>), dim3(nq * a.BH, a.splits), dim3(256), 0, st, a, sc);
  return hipGetLastError();
}

hipError_t launch_merge_bf16(const float* o_parts, const float* lse_parts, int parts, long long rows, int d,
                             __bf16* o, float* lse, hipStream_t st) {
  const int rpb = 256 / (d / 4);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (d == 64)
    hipLaunchKernelGGL((merge_kernel<64>), dim3(grid), dim3(256), 0, st, o_parts, lse_parts, parts, rows, o, lse);
  else
    hipLaunchKernelGGL((merge_kernel<128>), dim3(grid), dim3(256), 0, st, o_parts, lse_parts, parts, rows, o, lse);
  return hipGetLastError();
}

hipError_t launch_fwd_splitkv_bf16(const FwdArgs& a, hipStream_t stream) {
  const bool causal = a.causal != 0, sparse = a.mask != nullptr;
  hipError_t e;
  if (a.d == 64) {
    if (causal) e = sparse ? launch_splitkv_t<64, true, true>(a, stream) : launch_splitkv_t<64, true, false>(a, stream);
    else e = sparse ? launch_splitkv_t<64, false, true>(a, stream) : launch_splitkv_t<64, false, false>(a, stream);
  } else {
    if (causal) e = sparse ? launch_splitkv_t<128, true, true>(a, stream) : launch_splitkv_t<128, true, false>(a, stream);
    else e = sparse ? launch_splitkv_t<128, false, true>(a, stream) : launch_splitkv_t<128, false, false>(a, stream);
  }
  if (e != hipSuccess) return e;
  return launch_merge_bf16(a.o_part, a.lse_part, a.splits, (long long)a.BH * a.N, a.d, a.o, a.lse, stream);
}

}  // namespace fa
