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
//  * a negative scale is folded into Q's sign (exact in bf16), so the exponent uses |scale|;
//  * exponentials in base 2 with scale*log2(e) folded into one FMA; the running maximum is only
//    moved when a new score exceeds it by more than 2^8, so most tiles skip the O rescale (the
//    result is the same: numerator and denominator always share the offset).
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr float kRescaleThreshold = 8.0f;  // log2 units


// NW waves of 32 query rows each: BR = 32 NW rows per workgroup.  NW = 4 gives 128-row blocks
// (one mask block; two or three workgroups per CU); NW = 8 gives 256-row blocks with one
// workgroup per CU, so each K/V tile copied into LDS serves twice the query rows (half the
// L2 -> LDS copy traffic per flop).  Block-sparse masks need NW = 4.
template <int D, bool CAUSAL, bool SPARSE, bool SPLIT = false, int NW = 4>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : (D == 64 ? 3 : 2)) void fwd_bf16_kernel(FwdArgs a, Sched sc) {
  static_assert(NW == 4 || (NW == 8 && !SPARSE), "block-sparse masks need 128-row blocks");
  constexpr int BR = 32 * NW, BC = 64;
  constexpr int DC = D / 16;  // 16-wide contraction chunks over d
  constexpr int DB = D / 32;  // 32-row output blocks over d
  using KT = DmaTile<BC, D, NW>;  // K rows, read 16 bytes per lane
  using VT = DmaTile<BC, D, NW>;  // V rows, read transposed (ds_read_b64_tr_b16)

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
  // causal tiles of alternate cohorts walk the keys from the diagonal down (sched_descending);
  // the masks below depend only on each tile's first key, not on the order
  const bool desc = CAUSAL && !SPARSE && !SPLIT && sched_descending(sc, gridDim.x);
  auto tile_start = [&](int t) -> int {
    if (SPARSE) return (int)blist[t >> 1] * kMaskBlock + (t & 1) * BC;
    return (desc ? tend - 1 - t : tlo + t) * BC;
  };

  // ---- Q^T operand in registers (B operand: lane holds query q0 + 32w + c32, features 16c + 8h ..)
  const int qrow = q0 + 32 * w + c32;
  bf16x8 qreg[DC];
  load_qt_operand(Q, qrow, N, h, a.qsign, qreg);

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

  // S^T = K Q^T for two 32-key blocks; register r of half h holds key k0 + 32 kb + acc_row(r, h).
  // The two 32-key blocks alternate, so consecutive MFMAs are independent.
  auto scores = [&](const char* tk, f32x16(&s)[2]) {
    s[0] = zero16();
    s[1] = zero16();
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(lds_b128(tk + kaddr[c] + 32 * kb * D * 2), qreg[c], s[kb]);
  };
  // element masks: the causal diagonal and the key tail (only tiles that reach either).  With the
  // causal mask, register r of half h holds key base + c(r) with base = k0 + 32 kb + 8h and
  // c(r) = acc_row(r, 0), a constant; the key is masked when it is past N - 1 or past the lane's
  // query, i.e. when c(r) exceeds one per-lane threshold: one compare and one select per score on
  // the diagonal tiles.  Without it only the last tile is masked (the key tail).
  auto mask_tile = [&](f32x16(&s)[2], int k0) {
    if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0 + 32 * w)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if constexpr (CAUSAL) {
          const int thr = min(qrow, N - 1) - (k0 + 32 * kb + 8 * h);
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = acc_row(r, 0) > thr ? neg_inf() : s[kb][r];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (k0 + 32 * kb + acc_row(r, h) >= N) s[kb][r] = neg_inf();
        }
      }
    }
  };
  // online softmax: the running max (scaled log2 units) moves only when a score exceeds it by
  // more than 2^8; alpha is the factor that moves the accumulated O and sum onto the new max
  auto update_max = [&](const f32x16(&s)[2], float& m, float& alpha) {
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmax_nan(mt, s[kb][r]);
    mt = half_swap_max(mt) * sl;
    const float m_new = (mt > m + kRescaleThreshold) ? mt : m;
    alpha = (m_new == m) ? 1.f : fast_exp2(m - m_new);
    m = m_new;
  };

  // Software pipeline over key tiles (K runs one tile ahead of V, the scores and the max one
  // tile ahead of the exponentials):
  //   iteration t:  copies of K[t+2], V[t+1] in flight;
  //                 section 1: MFMAs of S[t+1] = K[t+1] Q^T, the exponentials of S[t] between them;
  //                 section 2: MFMAs of O += V[t] P[t], the row sums of P[t] and the max of S[t+1]
  //                            between them;  wait for the copies; barrier.
  // Each section pairs one matrix chain with VALU work that does not feed it, so the SIMD can
  // issue both.  K tiles alternate between kbuf0/kbuf1 and V tiles between vbuf0/vbuf1, so the
  // buffer a copy lands in during iteration t is never one read in iteration t.  The scores
  // alternate between sbuf[0] and sbuf[1] the same way, so no step copies registers.  The last
  // tile's section 1 multiplies the stale K buffer (in bounds; the result is discarded), which
  // keeps every section free of branches.
  f32x16 sbuf[2][2];
  float alpha = 1.f;
  if (ntiles > 0) {
    kdma.issue(K, N, kbuf0, tile_start(0), w);
    vdma.issue(V, N, vbuf0, tile_start(0), w);
    if (ntiles > 1) kdma.issue(K, N, kbuf1, tile_start(1), w);
  }
  wait_dma();
  __syncthreads();
  if (ntiles > 0) {
    scores(kbuf0, sbuf[0]);
    mask_tile(sbuf[0], tile_start(0));
    update_max(sbuf[0], m_used, alpha);
    alpha = 1.f;  // nothing accumulated yet
  }
  // every wave has read K[0] before step 0 copies K[2] over it (in later steps the barrier at
  // the end of the previous step orders the read of K[t] before the copy of K[t+2])
  if (ntiles > 2) lds_barrier();

  auto step = [&](int t, auto parity) {
    constexpr int par = decltype(parity)::value;  // t % 2
    char* const k_next = par ? kbuf0 : kbuf1;      // holds K[t+1] (stale K on the last tile)
    char* const k_free = par ? kbuf1 : kbuf0;      // held K[t]; receives K[t+2]
    char* const v_cur = par ? vbuf1 : vbuf0;       // holds V[t]
    char* const v_free = par ? vbuf0 : vbuf1;      // held V[t-1]; receives V[t+1]
    f32x16(&s_cur)[2] = sbuf[par];
    f32x16(&s_nxt)[2] = sbuf[par ^ 1];
    const bool has1 = t + 1 < ntiles, has2 = t + 2 < ntiles;
    if (has2) kdma.issue(K, N, k_free, tile_start(t + 2), w);
    if (has1) vdma.issue(V, N, v_free, tile_start(t + 1), w);

    if (wave_any(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
      lsum *= alpha;
    }
    const float msub = (m_used == neg_inf()) ? 0.f : m_used;

    // Wave priority per section (two waves of different workgroups share a SIMD): measured best
    // with section 1 first at d = 128, section 2 first at d = 64.
    __builtin_amdgcn_s_setprio(D == 128 ? 1 : 0);
    // section 1: S[t+1], and P[t] = exp2(S[t] * scale * log2(e) - m) in fp32 (kept in s_cur for
    // the row sum, so LSE carries fp32 error only) and rounded to bf16 for PV.
    // pk[2 kb + m2] holds keys k0 + 32 kb + 16 m2 + 8h + 0..7: one k-slot group of the PV MFMA.
    // Written out slot by slot in issue order (fenced, so the compiler keeps it): each MFMA is
    // followed by the FMAs of the next slot's scores, the exponentials of this slot's and the
    // bf16 conversion of the previous slot's; K operands are read four MFMAs ahead.
    constexpr int NS = 2 * DC;    // MFMAs (slots) in the section
    constexpr int EPS = 32 / NS;  // exponentials per slot
    auto sc = [&](int j) -> float { return s_cur[j >> 4][j & 15]; };
    auto kread = [&](int i) { return lds_b128(k_next + kaddr[i >> 1] + 32 * (i & 1) * D * 2); };
    bf16x8 pk[4];
    {
      bf16x8 kop[NS];
      float y[32];
      s_nxt[0] = zero16();
      s_nxt[1] = zero16();
#pragma unroll
      for (int i = 0; i < 4; ++i) kop[i] = kread(i);
#pragma unroll
      for (int j = 0; j < EPS; ++j) y[j] = __builtin_fmaf(sc(j), sl, -msub);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i + 4 < NS) kop[i + 4] = kread(i + 4);
        s_nxt[i & 1] = mfma32(kop[i], qreg[i >> 1], s_nxt[i & 1]);
#pragma unroll
        for (int e = 0; e < EPS; ++e)
          if ((i + 1) * EPS + e < 32) y[(i + 1) * EPS + e] = __builtin_fmaf(sc((i + 1) * EPS + e), sl, -msub);
#pragma unroll
        for (int e = 0; e < EPS; ++e) s_cur[(i * EPS + e) >> 4][(i * EPS + e) & 15] = fast_exp2(y[i * EPS + e]);
        if (i > 0) {
#pragma unroll
          for (int e = 0; e < EPS; ++e) pk[((i - 1) * EPS + e) >> 3][((i - 1) * EPS + e) & 7] = (__bf16)sc((i - 1) * EPS + e);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = 0; e < EPS; ++e) pk[((NS - 1) * EPS + e) >> 3][((NS - 1) * EPS + e) & 7] = (__bf16)sc((NS - 1) * EPS + e);
    }
    // pin P[t] here: without a use in this section the compiler sinks the exponentials past the
    // mask branch below, away from the MFMAs they are meant to run beside
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(pk[i]));
    asm volatile("" : "+v"(s_cur[0]), "+v"(s_cur[1]));
    __builtin_amdgcn_sched_barrier(0);

    if (has1) mask_tile(s_nxt, tile_start(t + 1));

    __builtin_amdgcn_s_setprio(D == 128 ? 0 : 1);
    // section 2: O^T += V^T P^T over the 64 keys (4 contraction chunks of 16; V^T read
    // transposed), the row sum of P[t] and the running max after S[t+1]
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const char* vb = v_cur + 16 * m * D * 2;
        oacc[db] = mfma32(join8(lds_tr4(vb + vaddr[0][db]), lds_tr4(vb + vaddr[1][db])), pk[m], oacc[db]);
      }
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[r & 3] += s_cur[kb][r];
    lsum += (part[0] + part[1]) + (part[2] + part[3]);
    asm volatile("" : "+v"(lsum));  // keep the row sums in this section as well
    {
      float m_nx = m_used, a_nx;
      update_max(s_nxt, m_nx, a_nx);
      asm volatile("" : "+v"(m_nx), "+v"(a_nx));  // computed here, whether or not used
      m_used = has1 ? m_nx : m_used;
      alpha = has1 ? a_nx : alpha;
    }
    // per MFMA: one transposed operand (two 8-byte reads, two MFMAs ahead), VALU work between
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      if (i < 4 * DB - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
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
// Wave-specialised forward ("ping-pong"), d = 128: the matrix work and the softmax of the pages'
// loop ([P2] "The Trick: Online Softmax") run in alternating phases on the two waves that share a
// SIMD, so that one wave's MFMAs overlap the other wave's exponentials (the interleaving of matrix
// products and softmax that "How FlashAttention Bypasses the GPU Memory Bottleneck to Enable
// Long-Context AI" credits for FlashAttention-3's throughput, here across the two waves of a
// SIMD instead of across warpgroups).
//
// One workgroup of 8 waves owns 256 query rows (32 per wave, Q^T held in registers as in
// fwd_bf16_kernel).  Waves w and w + 4 run on the same SIMD; wave group g = w / 4.  Every wave
// runs the same sequence of phases over its key tiles j = 0 .. T - 1 (64 keys each), one barrier
// after each phase:
//   M_j (matrix phase):  S[j] = K[j] Q^T (when j < T), O += V[j-1] P[j-1] (when j >= 1)
//   V_j (softmax phase): mask S[j], running max, rescale O, P[j] = exp2(S[j] - m), row sums
//   M_0 V_0 M_1 V_1 ... V_{T-1} M_T
// but group 1 starts one phase later (an idle phase first; group 0 ends with one), so in every
// phase one wave of each SIMD issues MFMAs while its partner issues the VALU work.  The matrix
// phase runs at raised wave priority (s_setprio), so its MFMAs issue first when both waves are
// ready.  K and V tiles are triple-buffered: K[j + 2] and V[j + 1] go into the buffers of K[j - 1]
// and V[j - 2], which group 1 last reads in global phase 2j - 1, and are first read in phase
// 2j + 4.  Each wave copies its share in global phase 2j (group 0 at the start of M_j, group 1 at
// the start of V_{j-1}) and waits for its previous share at the end of each V phase.
// Reached through flash_attn_fwd_pingpong; flash_attn_fwd keeps the in-wave interleave, which
// times faster on MI355X: here all operand reads of a tile fall into the matrix phase of each
// SIMD pair instead of spreading over the whole step.
template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd_pingpong_kernel(FwdArgs a, Sched sc) {
  constexpr int D = 128, NW = 8, BR = 32 * NW, BC = 64;
  constexpr int DC = D / 16, DB = D / 32;
  using KT = DmaTile<BC, D, NW>;

  __shared__ __attribute__((aligned(1024))) char kbuf[3][KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf[3][KT::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5,
            c32 = lane & 31;
  const int grp = w >> 2;
  const int N = a.N;
  int bh, qt;
  sched_decode(sc, gridDim.x, bh, qt);
  const int q0 = qt * BR;
  const size_t base = (size_t)bh * N * D;
  const __bf16* __restrict__ Q = a.q + base;
  const __bf16* __restrict__ K = a.k + base;
  const __bf16* __restrict__ V = a.v + base;
  int T = (N + BC - 1) / BC;
  if (CAUSAL) T = min(T, (min(q0 + BR, N) - 1) / BC + 1);
  // first key of the j-th tile visited: causal tiles of alternate cohorts walk the keys
  // downwards from the diagonal (sched_descending), as in fwd_bf16_kernel
  const bool desc = CAUSAL && sched_descending(sc, gridDim.x);
  auto kstart = [&](int j) -> int { return (desc ? T - 1 - j : j) * BC; };

  const int qrow = q0 + 32 * w + c32;
  bf16x8 qreg[DC];
  load_qt_operand(Q, qrow, N, h, a.qsign, qreg);
  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = zero16();
  float m_used = neg_inf(), lsum = 0.f;
  const float sl = a.scale_log2;

  int kaddr[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) kaddr[c] = KT::off(perm32(c32), 16 * c + 8 * h);
  int vaddr[2][DB];
  {
    const int g = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) vaddr[u][db] = KT::off4(8 * h + 4 * u + (j >> 2), 32 * db + 16 * g + 4 * (j & 3));
  }
  KT kdma, vdma;
  kdma.init(w, lane);
  vdma.init(w, lane);

  f32x16 s[2];   // S[j] of this wave's 32 queries: register r of half h holds key 64 j + 32 kb + acc_row(r, h)
  bf16x8 pk[4];  // P[j] as the PV B operand: pk[m] holds keys 64 j + 16 m + 8h + 0..7
#pragma unroll
  for (int m = 0; m < 4; ++m) pk[m] = zero_bf16x8();

  // matrix phase: 16 score MFMAs (HS) then 16 PV MFMAs (HP), each operand read from LDS four
  // MFMAs ahead of its use
  auto mphase = [&](auto hsc, auto hpc, const char* kb_, const char* vb_) __attribute__((always_inline)) {
    constexpr bool HS = decltype(hsc)::value, HP = decltype(hpc)::value;
    constexpr int I0 = HS ? 0 : 16, I1 = HP ? 32 : 16;
    auto rd = [&](int i) -> bf16x8 {
      if (i < 16) return lds_b128(kb_ + kaddr[i >> 1] + 32 * (i & 1) * D * 2);
      const int db = (i - 16) >> 2, m = (i - 16) & 3;
      const char* vb = vb_ + 16 * m * D * 2;
      return join8(lds_tr4(vb + vaddr[0][db]), lds_tr4(vb + vaddr[1][db]));
    };
    __builtin_amdgcn_s_setprio(1);
    if (HS) {
      s[0] = zero16();
      s[1] = zero16();
    }
    bf16x8 op[32];
#pragma unroll
    for (int i = I0; i < I0 + 4 && i < I1; ++i) op[i] = rd(i);
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      if (i + 4 < I1) op[i + 4] = rd(i + 4);
      if (i < 16)
        s[i & 1] = mfma32(op[i], qreg[i >> 1], s[i & 1]);
      else
        oacc[(i - 16) >> 2] = mfma32(op[i], pk[(i - 16) & 3], oacc[(i - 16) >> 2]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // softmax phase of tile j: masks, running maximum (moved only past a 2^8 margin, as in
  // fwd_bf16_kernel), rescale of O, P = exp2(S scale log2(e) - m) in fp32 for the row sums and
  // as bf16 for PV
  auto vphase = [&](int j) __attribute__((always_inline)) {
    const int k0 = kstart(j);
    if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0 + 32 * w)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if constexpr (CAUSAL) {
          const int thr = min(qrow, N - 1) - (k0 + 32 * kb + 8 * h);
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = acc_row(r, 0) > thr ? neg_inf() : s[kb][r];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (k0 + 32 * kb + acc_row(r, h) >= N) s[kb][r] = neg_inf();
        }
      }
    }
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmax_nan(mt, s[kb][r]);
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
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
      const float p = fast_exp2(__builtin_fmaf(s[jj >> 4][jj & 15], sl, -msub));
      part[jj & 3] += p;
      pk[jj >> 3][jj & 7] = (__bf16)p;
    }
    lsum += (part[0] + part[1]) + (part[2] + part[3]);
  };
  // this wave's share of the copies of K[i] and V[i - 1] into buffers i % 3 and (i - 1) % 3 (tiles
  // past the end are skipped); returns the copy instructions issued
  auto prefetch = [&](int i, auto rc) -> int {
    constexpr int r = decltype(rc)::value;  // i % 3
    int n = 0;
    if (i < T) {
      kdma.issue(K, N, kbuf[r], kstart(i), w);
      n += KT::CH;
    }
    if (i - 1 < T) {
      vdma.issue(V, N, vbuf[(r + 2) % 3], kstart(i - 1), w);
      n += KT::CH;
    }
    return n;
  };
  // end of a softmax phase: the previous batch of this wave's copies has landed (the latest, n
  // instructions, may stay in flight); then the barrier that publishes them
  auto vphase_end = [&](int n) {
    if (n == 2 * KT::CH)
      wait_vm<2 * KT::CH>();
    else if (n == KT::CH)
      wait_vm<KT::CH>();
    else
      wait_vm<0>();
    lds_barrier();
  };
  auto phase_end = []() { asm volatile("s_barrier" ::: "memory"); };

  // unit j (buffers j % 3 fixed at compile time): M_j, then V_j when j < T.  Group 0 copies K[j+2]
  // and V[j+1] as it starts M_j; group 1 copies K[j+3] and V[j+2] as it starts V_j.
  auto unit = [&](int j, auto rc, auto hsc, auto hpc) __attribute__((always_inline)) {
    constexpr int r = decltype(rc)::value;
    constexpr bool HS = decltype(hsc)::value;
    int n = 0;
    if (grp == 0) n = prefetch(j + 2, std::integral_constant<int, (r + 2) % 3>{});
    mphase(hsc, hpc, kbuf[r], vbuf[(r + 2) % 3]);
    phase_end();
    if (HS) {
      if (grp != 0) n = prefetch(j + 3, std::integral_constant<int, r>{});
      vphase(j);
      vphase_end(n);
    }
  };

  // prologue: K[0], K[1], V[0] by every wave, and group 1's share of K[2], V[1] (group 0 copies
  // its share at the start of M_0); then group 1's idle phase
  kdma.issue(K, N, kbuf[0], kstart(0), w);
  if (T > 1) kdma.issue(K, N, kbuf[1], kstart(1), w);
  vdma.issue(V, N, vbuf[0], kstart(0), w);
  wait_vm<0>();
  lds_barrier();
  if (grp != 0) {
    const int n = prefetch(2, std::integral_constant<int, 2>{});
    (void)n;
    phase_end();
  }

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using Y = std::true_type;
  using F = std::false_type;
  unit(0, I0{}, Y{}, F{});
  int j = 1;
  for (; j + 2 < T; j += 3) {
    unit(j, I1{}, Y{}, Y{});
    unit(j + 1, I2{}, Y{}, Y{});
    unit(j + 2, I0{}, Y{}, Y{});
  }
  if (j < T) {  // j % 3 == 1 here; at most two full units remain before unit T
    unit(j, I1{}, Y{}, Y{});
    ++j;
    if (j < T) {
      unit(j, I2{}, Y{}, Y{});
      ++j;
    }
  }
  switch (T % 3) {  // unit T: the last PV only
    case 0: unit(T, I0{}, F{}, Y{}); break;
    case 1: unit(T, I1{}, F{}, Y{}); break;
    default: unit(T, I2{}, F{}, Y{}); break;
  }
  if (grp == 0) phase_end();  // group 0's idle phase at the end

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
  constexpr int NW = (D == 128 && !S) ? 8 : 4;  // 256-row blocks at d = 128 (1-2% faster than 128-row)
  constexpr int BR = 32 * NW;
  const int nq = (a.N + BR - 1) / BR;
  static const int slots = xcd_slots(reinterpret_cast<const void*>(&fwd_bf16_kernel<D, C, S, false, NW>), 64 * NW);
  const Sched sc = make_sched(nq, a.BH, /*heavy_last_tile=*/1, slots, /*uneven=*/C || S, /*alternate=*/C && !S);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, C, S, false, NW>), dim3(nq * a.BH), dim3(64 * NW), 0, st, a, sc);
  return hipGetLastError();
}

template <bool C>
static hipError_t launch_pingpong_t(const FwdArgs& a, hipStream_t st) {
  const int nq = (a.N + 255) / 256;
  static const int slots = xcd_slots(reinterpret_cast<const void*>(&fwd_pingpong_kernel<C>), 512);
  const Sched sc = make_sched(nq, a.BH, /*heavy_last_tile=*/1, slots, /*uneven=*/C, /*alternate=*/C);
  hipLaunchKernelGGL((fwd_pingpong_kernel<C>), dim3(nq * a.BH), dim3(512), 0, st, a, sc);
  return hipGetLastError();
}

hipError_t launch_fwd_pingpong_bf16(const FwdArgs& a, hipStream_t stream) {
  return a.causal ? launch_pingpong_t<true>(a, stream) : launch_pingpong_t<false>(a, stream);
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
  const Sched sc = make_sched(nq, a.BH, /*heavy_last_tile=*/1, slots, /*uneven=*/C || S);
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
