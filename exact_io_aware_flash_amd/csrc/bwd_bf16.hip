// Backward pass, bf16 inputs/outputs, fp32 accumulation, for gfx950.
//
// The pages keep only the per-row softmax statistic from the forward pass and recompute the
// rest tile by tile ([P3] "How FlashAttention Eliminates Transformer Memory Bottlenecks",
// "Innovation #3: Strategic recomputation in the backward pass").  With LSE saved,
// P = exp(scale Q K^T - LSE) needs no running maximum.  Gradients of L = sum(O * dO):
//   D = rowsum(dO * O)            (pre-pass; equals rowsum(P * dP))
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dK = scale dS^T Q,  dQ = scale dS K.
//
// Three kernels on one stream:
//  1. bwd_delta:  D per row (bandwidth-bound, 16-byte loads, shuffle reduction).
//  2. bwd_dkdv:   one workgroup per (b*h, 128-key block).  d = 128: 8 waves, two per 32 keys
//                 (one computes P and dV with K in registers, the other dP, dS and dK with V in
//                 registers, P passing between them through LDS); d = 64: 4 waves, one per 32
//                 keys, two workgroups per CU.  Q and dO tiles of 128 rows are copied
//                 global -> LDS asynchronously (double-buffered), LSE and D beside them.
//                 S = Q K^T puts one key per lane and 16 queries in registers, the A-operand
//                 shape of dV = P^T dO and dK = dS^T Q; their B operands (dO and Q with queries as
//                 the contraction index) are read from the same tiles with transposing reads.
//  3. bwd_dq:     one workgroup per (b*h, 128-query block), K and V tiles of 64 keys copied
//                 asynchronously into LDS: S^T = K Q^T and dP^T = V dO^T give one query per lane
//                 (the B-operand shape of dQ^T = K^T dS^T); K^T is read transposed from the K tile.
//                 The tile's two 32-key blocks are software-pipelined (the exponentials and dS of
//                 one block between the MFMAs of the other).
// dQ is produced without atomics, so every output element is written once and results are
// bitwise reproducible run to run.
// A negative scale is folded into the sign of the operand each kernel holds in registers for S
// (K in dK/dV, Q in dQ; exact in bf16), so P = exp2(|scale| log2(e) S' - LSE log2(e)) with
// S' = sign(scale) Q K^T; dK and dQ are multiplied by the signed scale at the end.
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

namespace {

// ------------------------------------------------------------------------------------------ D
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                        float* __restrict__ delta, long rows) {
  constexpr int EPL = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int TPR = D / EPL;         // threads per row (power of two)
  constexpr int RPB = 256 / TPR;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const uint4 ov = *reinterpret_cast<const uint4*>(o + row * D + part * EPL);
    const uint4 dv = *reinterpret_cast<const uint4*>(dout + row * D + part * EPL);
    const T* op = reinterpret_cast<const T*>(&ov);
    const T* dp = reinterpret_cast<const T*>(&dv);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc += (float)op[e] * (float)dp[e];
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && part == 0) delta[row] = acc;
}

// --------------------------------------------------------------------------- dK, dV at d = 64
// One workgroup of 4 waves per (b*h, 128-key block), each wave doing all the work on 32 keys
// (K and V both in registers); two workgroups fit on a CU, so each SIMD still runs two waves.
// Short per-block tile lists (small N, block-sparse masks) favour this form over the paired
// waves below, whose phase pipeline has a fill and a drain per workgroup.
template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_wave_kernel(BwdArgs a, Sched sc) {
  static_assert(D == 64, "the single-wave dK/dV kernel serves d = 64");
  constexpr int BKV = 128, BQ = 128;  // one mask block of keys against one of queries per step
  constexpr int NH = BQ / 32;          // 32-query parts of a query tile
  constexpr int DC = D / 16, DB = D / 32;
  using QT = DmaTile<BQ, D>;  // Q or dO rows (read row-wise and transposed)

  __shared__ __attribute__((aligned(1024))) char qbuf0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char qbuf1[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char obuf0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char obuf1[QT::BYTES];
  __shared__ __attribute__((aligned(16))) float lbuf[2][BQ];
  __shared__ __attribute__((aligned(16))) float dbuf[2][BQ];
  __shared__ unsigned short blist[SPARSE ? kMaxMaskBlocks : 1];
  __shared__ int bcount;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, c32 = lane & 31;
  const int N = a.N;
  int bh, kt;
  sched_decode(sc, gridDim.x, bh, kt);
  const int k0 = kt * BKV;
  const int k0w = k0 + 32 * w;
  const size_t base = (size_t)bh * N * D;
  const size_t rbase = (size_t)bh * N;
  const __bf16* __restrict__ Qh = a.q + base;
  const __bf16* __restrict__ Oh = a.dout + base;

  // ---- query tiles (of BQ rows) that see this key block
  const int nqt = (N + BQ - 1) / BQ;
  int q_first = 0, ntiles = nqt;
  if (CAUSAL) {
    q_first = k0 / BQ;
    ntiles = nqt - q_first;
  }
  if (SPARSE) {
    if (w == 0) {
      const int cnt = build_block_list(a.mask, a.nb, kt, true, CAUSAL ? kt : 0, a.nb, blist, lane);
      if (lane == 0) bcount = cnt;
    }
    __syncthreads();
    const int cnt = bcount;
    ntiles = cnt;  // one query tile per mask block
  }
  auto tile_start = [&](int t) -> int {
    if (SPARSE) return (int)blist[t] * kMaskBlock;
    return (q_first + t) * BQ;
  };

  // ---- this lane's key: K and V rows as B operands (features 16c + 8h ..)
  const int key = k0w + c32;
  bf16x8 kreg[DC], vreg[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    if (key < N) {
      kreg[c] = xor_sign(*reinterpret_cast<const bf16x8*>(a.k + base + (size_t)key * D + 16 * c + 8 * h), a.ssign);
      vreg[c] = *reinterpret_cast<const bf16x8*>(a.v + base + (size_t)key * D + 16 * c + 8 * h);
    } else {
      kreg[c] = zero_bf16x8();
      vreg[c] = zero_bf16x8();
    }
  }
  f32x16 dvacc[DB], dkacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dvacc[i] = zero16();
    dkacc[i] = zero16();
  }
  const float sl = a.scale_log2;

  // ---- per-lane LDS addresses
  // A operands (Q, dO rows): row 32 s + perm32(c32) (32 s added per use), features 16c + 8h ..
  int raddr[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) raddr[c] = QT::off(perm32(c32), 16 * c + 8 * h);
  // B operands (dO^T, Q^T: queries as the contraction index), transposed read u of feature
  // block db: lane j of its 16-lane group addresses query row 8h + 4u + j/4 (+ 32 s + 16 mm)
  int taddr[2][DB];
  {
    const int g = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) taddr[u][db] = QT::off4(8 * h + 4 * u + (j >> 2), 32 * db + 16 * g + 4 * (j & 3));
  }

  QT qdma, odma;
  qdma.init(w, lane);
  odma.init(w, lane);
  float lpre = 0.f, dlpre = 0.f;
  auto rowstats_load = [&](int q0) {
    if (tid < BQ) {
      const int qr = q0 + tid;
      // rows past N, or rows that see no key, get +inf so that P = 0
      const float l = qr < N ? a.lse[rbase + qr] : neg_inf();
      lpre = (l == neg_inf()) ? __builtin_huge_valf() : l * kLog2e;
      dlpre = qr < N ? a.delta[rbase + qr] : 0.f;
    }
  };
  auto rowstats_store = [&](int buf) {
    if (tid < BQ) {
      lbuf[buf][tid] = lpre;
      dbuf[buf][tid] = dlpre;
    }
  };

  if (ntiles > 0) {
    const int q0 = tile_start(0);
    qdma.issue(Qh, N, qbuf0, q0, w);
    odma.issue(Oh, N, obuf0, q0, w);
    rowstats_load(q0);
    rowstats_store(0);
  }
  wait_dma();
  __syncthreads();

  // S = Q K^T and dP = dO V^T of 32-query part s (rows 32 s .. 32 s + 31 of the tile, queries
  // qs ..): register r of half h holds query 32 s + acc_row(r, h) of the tile, key `key`.
  // Accumulated in VGPRs by inline-asm MFMAs (the compiler's MFMAs may keep their accumulators in
  // AGPRs, where each VALU read would cost a copy), operand reads two MFMA pairs ahead of their
  // use; `hook(c)` runs after MFMA pair c in the same fenced slot (independent VALU work, issued
  // while the MFMAs run).  `mask`: S starts at -inf where the pair (query, key) is masked (the key
  // tail, and the causal diagonal for query part qs), instead of 0, so that P = exp(S - LSE) is 0
  // there with no VALU work on the scores; the MFMA reading that VALU-written accumulator needs 2
  // wait states.  The asm is opaque to the compiler's hazard tracking: a VALU read of S or dP
  // needs 14 wait states after the MFMA that wrote it (gfx950), given after the chain.
  auto sp_chain = [&](const char* tq, const char* to, int s, f32x16& sacc, f32x16& pacc, bool mask, int qs,
                      auto hook) __attribute__((always_inline)) {
    bf16x8 qa[DC], oa[DC];
    auto rd = [&](int c) {
      qa[c] = lds_b128(tq + raddr[c] + 32 * s * D * 2);
      oa[c] = lds_b128(to + raddr[c] + 32 * s * D * 2);
    };
    rd(0);
    rd(1);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      if (c + 2 < DC) rd(c + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (c == 0) {
        if (mask) {
          // element r is query qs + 8h + 16 (r / 8) + r % 8: masked when 16 (r / 8) + r % 8 < thr
          const int thr = key >= N ? 32 : (CAUSAL ? key - qs - 8 * h : 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[r] = 16 * (r >> 3) + (r & 7) < thr ? neg_inf() : 0.f;
          asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc) : "v"(qa[0]), "v"(kreg[0]));
        } else {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(sacc) : "v"(qa[0]), "v"(kreg[0]));
        }
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(pacc) : "v"(oa[0]), "v"(vreg[0]));
      } else {
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc) : "v"(qa[c]), "v"(kreg[c]));
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(pacc) : "v"(oa[c]), "v"(vreg[c]));
      }
      hook(c);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(sacc), "+v"(pacc));  // 16 wait states
  };

  // Score elements 4 qq .. 4 qq + 3 of a part are queries 16 (qq / 2) + 8h + 4 (qq % 2) + 0..3;
  // pp / dsp[mm] (bf16 A operands) hold queries 16 mm + 8h + 0..7.  Rows past N, and rows that
  // see no key, have LSE = +inf here, so P = 0 there.
  auto stat4 = [&](const float* rows, int s, int qq) -> f32x4 {
    return *reinterpret_cast<const f32x4*>(rows + 32 * s + 16 * (qq >> 1) + 8 * h + 4 * (qq & 1));
  };
  // P = exp(S - LSE) of quarter qq, written over S in place (fp32, for dS) and as bf16 into pp
  auto p_quarter = [&](f32x16& x, const f32x4& l, int qq, bf16x8(&pp)[2]) __attribute__((always_inline)) {
    const int mm = qq >> 1, e0 = 4 * (qq & 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 8 * mm + e0 + e;
      const float p = fast_exp2(__builtin_fmaf(x[r], sl, -l[e]));
      x[r] = p;
      pp[mm][e0 + e] = (__bf16)p;
    }
  };
  // dS = P (dP - D) of quarter qq, from P (in x) and dP (in y)
  auto ds_quarter = [&](const f32x16& x, const f32x16& y, const f32x4& d, int qq, bf16x8(&dsp)[2])
      __attribute__((always_inline)) {
    const int mm = qq >> 1, e0 = 4 * (qq & 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 8 * mm + e0 + e;
      dsp[mm][e0 + e] = (__bf16)(x[r] * (y[r] - d[e]));
    }
  };

  // dV += P^T dO, then dK += dS^T Q, for part s (contraction over its 32 queries, two chunks of
  // 16; MFMA i takes feature block i / 2 and chunk i % 2).  Each MFMA takes one transposed B
  // operand (two 8-byte transposing reads), read two MFMAs ahead.  dS of quarter i is computed in
  // the slot of dV MFMA i (D read one slot ahead), so the dK MFMAs find it complete.
  auto dvdk = [&](const char* tq, const char* to, int s, const bf16x8(&pp)[2], const f32x16& x, const f32x16& y,
                  const float* Ds) __attribute__((always_inline)) {
    static_assert(DB == 2, "four MFMAs per product at d = 64");
    bf16x8 ob[4], qb[4], dsp[2];
    auto trd = [&](const char* t, int i) -> bf16x8 {
      const int db = i >> 1, roff = (32 * s + 16 * (i & 1)) * D * 2;
      return join8(lds_tr4(t + roff + taddr[0][db]), lds_tr4(t + roff + taddr[1][db]));
    };
    ob[0] = trd(to, 0);
    ob[1] = trd(to, 1);
    f32x4 d = stat4(Ds, s, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i + 2 < 4) ob[i + 2] = trd(to, i + 2);
      else qb[i - 2] = trd(tq, i - 2);
      const f32x4 dc = d;
      if (i + 1 < 4) d = stat4(Ds, s, i + 1);
      dvacc[i >> 1] = mfma32(pp[i & 1], ob[i], dvacc[i >> 1]);
      ds_quarter(x, y, dc, i, dsp);
      if (i & 1) asm volatile("" : "+v"(dsp[i >> 1]));  // computed in this slot
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i + 2 < 4) qb[i + 2] = trd(tq, i + 2);
      dkacc[i >> 1] = mfma32(dsp[i & 1], qb[i], dkacc[i >> 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One query tile, its four 32-query parts software-pipelined within the wave: the S / dP MFMAs
  // of part s + 1 carry P of part s in their slots (a quarter of the part's elements per MFMA
  // pair, the LSE read one slot ahead), then the dV MFMAs of part s carry its dS, then its dK
  // MFMAs run.  Every part is computed, also one that lies wholly above the causal diagonal or
  // past N: its masks (or its LSE of +inf) make P and dS zero, so it adds nothing.
  auto step = [&](int t, auto parity) {
    constexpr int par = decltype(parity)::value;
    const char* tq = par ? qbuf1 : qbuf0;
    const char* to = par ? obuf1 : obuf0;
    const int q0 = tile_start(t);
    const bool has_next = t + 1 < ntiles;
    if (has_next) {
      const int qn = tile_start(t + 1);
      qdma.issue(Qh, N, par ? qbuf0 : qbuf1, qn, w);
      odma.issue(Oh, N, par ? obuf0 : obuf1, qn, w);
      rowstats_load(qn);
    }
    const float* Ls = lbuf[par];
    const float* Ds = dbuf[par];
    // parts that reach the key tail or the causal diagonal of this wave's keys
    auto part_mask = [&](int qs) -> bool { return (k0w + 32 > N) || (CAUSAL && qs < k0w + 31); };
    f32x16 sv[2], pv[2];  // S (then P) and dP of part s in sv / pv[s & 1]
    sp_chain(tq, to, 0, sv[0], pv[0], part_mask(q0), q0, [](int) {});
#pragma unroll
    for (int s = 0; s < NH; ++s) {
      bf16x8 pp[2];
      f32x16& x = sv[s & 1];
      f32x4 l = stat4(Ls, s, 0);
      auto quarter = [&](int qq) __attribute__((always_inline)) {
        const f32x4 lc = l;
        if (qq + 1 < 4) l = stat4(Ls, s, qq + 1);
        p_quarter(x, lc, qq, pp);
        if (qq & 1) asm volatile("" : "+v"(pp[qq >> 1]));  // computed in this slot
      };
      if (s + 1 < NH) {
        const int qs1 = q0 + 32 * (s + 1);
        sp_chain(tq, to, s + 1, sv[(s + 1) & 1], pv[(s + 1) & 1], part_mask(qs1), qs1, quarter);
      } else {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) quarter(qq);
      }
      dvdk(tq, to, s, pp, x, pv[s & 1], Ds);
    }
    if (has_next) rowstats_store(par ^ 1);
    wait_dma();
    __syncthreads();
  };

  for (int t = 0; t < ntiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: lane holds feature 32 db + c32 of keys k0w + 8 g + 4 h + e (register 4 g + e)
  const float scale = a.scale;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = k0w + 8 * (r >> 2) + 4 * h + (r & 3);
      if (kr < N) {
        const size_t off = base + (size_t)kr * D + 32 * db + c32;
        a.dv[off] = (__bf16)dvacc[db][r];
        a.dk[off] = (__bf16)(dkacc[db][r] * scale);
      }
    }
}

// ------------------------------------------------------------------------------------- dK, dV
// One workgroup of 8 waves per (b*h, 128-key block).  Waves w and w + 4 own the same 32 keys
// k0 + 32 (w % 4) .. + 31 and split the work on them (two waves per SIMD, so each one's LDS and
// VALU latency has the other's MFMAs to hide behind):
//   P wave  (w < 4):  S = Q K^T, P = exp(S - LSE) with the masks, dV += P^T dO   (K in registers)
//   dS wave (w >= 4): dP = dO V^T, dS = P (dP - D), dK += dS^T Q              (V in registers)
// P goes from one to the other through LDS as bf16, the values dV uses.  Query tiles of 128 rows
// are split into four 32-query parts; the dS wave runs one part behind: in phase s of tile t the
// P waves handle part s and the dS waves part s - 1 (in phase 0, part 3 of tile t - 1), with one
// barrier per phase.  Q and dO tiles are double-buffered; the copy of tile t + 1 starts in
// phase 1 of tile t, once the dS waves are done with tile t - 1.
template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(512) void bwd_dkdv_kernel(BwdArgs a, Sched sc) {
  constexpr int BKV = 128, BQ = 128;  // one mask block of keys against one of queries per tile
  constexpr int NH = BQ / 32;          // 32-query parts of a query tile
  constexpr int DC = D / 16, DB = D / 32;
  using QT = DmaTile<BQ, D, 8>;  // Q or dO rows (read row-wise and transposed)

  __shared__ __attribute__((aligned(1024))) char qbuf0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char qbuf1[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char obuf0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char obuf1[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char pbuf[4][2][2048];  // P of one part, per key group and phase parity
  __shared__ __attribute__((aligned(16))) float lbuf[2][BQ];
  __shared__ __attribute__((aligned(16))) float dbuf[2][BQ];
  __shared__ unsigned short blist[SPARSE ? kMaxMaskBlocks : 1];
  __shared__ int bcount;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w & 3;     // key group: keys k0 + 32 grp ..
  const bool dsw = w >= 4;   // dS wave
  const int N = a.N;
  int bh, kt;
  sched_decode(sc, gridDim.x, bh, kt);
  const int k0 = kt * BKV;
  const int k0w = k0 + 32 * grp;
  const size_t base = (size_t)bh * N * D;
  const size_t rbase = (size_t)bh * N;
  const __bf16* __restrict__ Qh = a.q + base;
  const __bf16* __restrict__ Oh = a.dout + base;

  // ---- query tiles (of BQ rows) that see this key block
  const int nqt = (N + BQ - 1) / BQ;
  int q_first = 0, ntiles = nqt;
  if (CAUSAL) {
    q_first = k0 / BQ;
    ntiles = nqt - q_first;
  }
  if (SPARSE) {
    if (w == 0) {
      const int cnt = build_block_list(a.mask, a.nb, kt, true, CAUSAL ? kt : 0, a.nb, blist, lane);
      if (lane == 0) bcount = cnt;
    }
    __syncthreads();
    ntiles = bcount;  // one query tile per mask block
  }
  auto tile_start = [&](int t) -> int {
    if (SPARSE) return (int)blist[t] * kMaskBlock;
    return (q_first + t) * BQ;
  };

  // ---- this lane's key: its K (P wave) or V (dS wave) row as B operands (features 16c + 8h ..)
  const int key = k0w + c32;
  const __bf16* __restrict__ kvsrc = (dsw ? a.v : a.k) + base;
  const uint32_t ksign = dsw ? 0u : a.ssign;  // the sign of scale rides on K (P wave only)
  bf16x8 kv[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c)
    kv[c] = key < N ? xor_sign(*reinterpret_cast<const bf16x8*>(kvsrc + (size_t)key * D + 16 * c + 8 * h), ksign)
                    : zero_bf16x8();
  f32x16 acc[DB];  // dV (P wave) or dK / scale (dS wave)
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = zero16();
  const float sl = a.scale_log2;

  // ---- per-lane LDS addresses
  // A operands (Q, dO rows): row 32 s + perm32(c32) (32 s added per use), features 16c + 8h ..
  int raddr[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) raddr[c] = QT::off(perm32(c32), 16 * c + 8 * h);
  // B operands (dO^T, Q^T: queries as the contraction index), transposed read u of feature
  // block db: lane j of its 16-lane group addresses query row 8h + 4u + j/4 (+ 32 s + 16 mm)
  int taddr[2][DB];
  {
    const int g = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) taddr[u][db] = QT::off4(8 * h + 4 * u + (j >> 2), 32 * db + 16 * g + 4 * (j & 3));
  }

  QT qdma, odma;
  qdma.init(w, lane);
  odma.init(w, lane);
  // LSE and D of the next tile: loaded when its copy starts, used only when stored (at the end
  // of the tile), so that no wait on the loads holds up the copies issued before them
  // (by the first two P waves only; rows past N load row N - 1 and are replaced when stored, so
  // that nothing right after the loads waits for them)
  float lraw = 0.f, draw = 0.f;
  bool rlive = false;
  auto rowstats_load = [&](int q0) {
    if (!dsw && tid < BQ) {
      const int qr = q0 + tid;
      rlive = qr < N;
      const size_t r = rbase + min(qr, N - 1);
      lraw = a.lse[r];
      draw = a.delta[r];
    }
  };
  auto rowstats_store = [&](int buf) {
    if (!dsw && tid < BQ) {
      // rows past N, or rows that see no key, get +inf so that P = 0
      lbuf[buf][tid] = (!rlive || lraw == neg_inf()) ? __builtin_huge_valf() : lraw * kLog2e;
      dbuf[buf][tid] = rlive ? draw : 0.f;
    }
  };

  if (ntiles > 0) {
    const int q0 = tile_start(0);
    qdma.issue(Qh, N, qbuf0, q0, w);
    odma.issue(Oh, N, obuf0, q0, w);
    rowstats_load(q0);
    wait_dma();
    rowstats_store(0);
  }
  __syncthreads();

  // X B^T for query part s, X rows read from tile `t` (Q or dO), B = this wave's K or V rows:
  // register r of half h holds query 32 s + acc_row(r, h) of the tile, key `key`.  Accumulated
  // in VGPRs by inline-asm MFMAs (the compiler's MFMAs may keep their accumulators in AGPRs,
  // where each VALU read would cost a copy).  Operand reads run two MFMAs ahead; `hook(c)` runs
  // after MFMA c in the same fenced slot (independent VALU work, issued while the MFMA runs).
  // The accumulator starts at zero, or (`cinit`) at a per-row vector read from LDS (the dS
  // waves start dP at -D), or (`mask`) at -inf where the pair (query, key) is masked (the key
  // tail, and the causal diagonal for query block row qs), so that P = exp(S - LSE) is 0 there
  // without further VALU work.  The asm is opaque to the compiler's hazard tracking: a VALU read
  // of the result needs 14 wait states after the last MFMA (gfx950), given at the end, and an
  // MFMA reading a VALU result as its accumulator needs 2, given before it.
  auto chain = [&](const char* t, int s, f32x16& x, bool mask, int qs, const float* cinit, auto hook)
      __attribute__((always_inline)) {
    bf16x8 op[DC];
    auto rd = [&](int c) { op[c] = lds_b128(t + raddr[c] + 32 * s * D * 2); };
    rd(0);
    rd(1);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      if (c + 2 < DC) rd(c + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (c == 0) {
        if (cinit) {
          // accumulator initialised from LDS: 16 rows 16 (r / 8) + 8h + r % 8 of a row vector
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(cinit + 16 * (i >> 1) + 8 * h + 4 * (i & 1));
#pragma unroll
            for (int j = 0; j < 4; ++j) x[4 * i + j] = v[j];
          }
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(x) : "v"(op[0]), "v"(kv[0]));
        } else if (mask) {
          // element r is query qs + 8h + 16 (r / 8) + r % 8: masked when 16 (r / 8) + r % 8 < thr
          const int thr = key >= N ? 32 : (CAUSAL ? key - qs - 8 * h : 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = 16 * (r >> 3) + (r & 7) < thr ? neg_inf() : 0.f;
          asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(x) : "v"(op[0]), "v"(kv[0]));
        } else {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(x) : "v"(op[0]), "v"(kv[0]));
        }
      } else {
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(x) : "v"(op[c]), "v"(kv[c]));
      }
      hook(c);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x));  // 16 wait states
  };

  // acc += X^T Y for query part s: X = P or dS of the part (A operands, one key per lane and
  // queries 16 mm + 8h .. as the contraction index), Y = dO or Q rows of the part, read from
  // tile `t` with transposing reads (two 8-byte reads per MFMA, kept four MFMAs ahead); MFMAs
  // on the same accumulator DB apart (a region of its own, so that its scheduling groups take
  // only its own reads)
  auto accumulate = [&](const char* t, int s, const bf16x8(&x)[2]) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int roff = (32 * s + 16 * mm) * D * 2;
        acc[db] = mfma32(x[mm], join8(lds_tr4(t + roff + taddr[0][db]), lds_tr4(t + roff + taddr[1][db])), acc[db]);
      }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 2 * DB - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // copy of tile t + 1 into the other buffers (from phase 2 of tile t, once no wave reads tile
  // t - 1 any more), by all waves
  // (the buffer is a compile-time choice: copies into an LDS address the compiler cannot place
  // make it wait for them before every later LDS read)
  auto prefetch = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int qn = tile_start(t + 1);
    qdma.issue(Qh, N, buf ? qbuf1 : qbuf0, qn, w);
    odma.issue(Oh, N, buf ? obuf1 : obuf0, qn, w);
    rowstats_load(qn);
  };
  // end of tile t: the next tile's LSE and D stored, its copies landed (a barrier follows)
  auto finish_tile = [&](bool has_next, int buf) {
    if (has_next) rowstats_store(buf);
    wait_dma();
  };
  auto tile_mask = [&](int q0) -> bool {
    // tiles touching the key tail or the causal diagonal; queries past N need no mask (their
    // LSE is +inf, so P = 0)
    return (k0 + BKV > N) || (CAUSAL && q0 < k0 + BKV - 1);
  };

  // Parts are never skipped: the masks give P = 0 wherever a part sees no key (and rows past N
  // have P = 0 through their LSE), and the phase barrier would keep the group waiting anyway.
  //
  // Number the 32-query parts g = 4 t + s over the tiles.  In phase g (one barrier each):
  //   P wave:  S MFMAs of part g, with the exponentials of part g - 1 in their slots; P of part
  //            g - 1 to LDS; dV MFMAs of part g - 1
  //   dS wave: dP MFMAs of part g - 1, with dS of part g - 2 (P of g - 2 from LDS) in their
  //            slots; dK MFMAs of part g - 2
  // Tile t - 1 is last read in phase 1 of tile t (dK of its part 3), so the copy of tile t + 1
  // into its buffers starts in phase 2.  After the last tile, one more phase with a barrier
  // (P wave: exponentials and dV of the last part) and one without (dS wave: its last part).
  // Pairs j = 0..7 (elements 2j, 2j + 1) of a part's scores take chain slots SKIP .. DC - 1: the
  // first slots give the LDS reads the pairs need (P, the row statistics) time to land.
  constexpr int SKIP = DC / 4;
  auto pair_slot = [](int j) constexpr { return SKIP + j * (DC - SKIP) / 8; };
  // Row statistics (LSE or D) of a part reach the lanes through one 4-byte LDS read per lane: lane
  // 16 i + k holds the value of row 16 (k / 8) + 8 (i / 2) + k % 8 of the part, and a DPP row
  // broadcast of lane k within each row of 16 lanes then gives every lane of half h the value of
  // score element r = k (row 16 (r / 8) + 8h + r % 8).
  // (the lane's byte offset is formed once, so that each read is the array plus two offsets: a
  // longer chain of address steps loses the compiler's knowledge of which LDS array is read, and
  // it then waits for every copy into LDS in flight before the read)
  const int stat_off = 4 * (16 * ((lane & 15) >> 3) + 8 * h + (lane & 7));
  auto stat_load = [&](const float* rows, int s) -> float {
    return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(rows) + 128 * s + stat_off);
  };
  auto stat_of = [](float v, int r) __attribute__((always_inline)) -> float { return row_bcast(v, r); };
  if (!dsw) {
    f32x16 sv[2];  // S of part g in sv[g & 1]
    // phase with S of part s of tile buffers tq (when HS) and exponentials / dV of part s_e of
    // buffers to_e (when HE)
    auto p_phase = [&](auto hsc, auto hec, const char* tq, int s, bool mask, int qs, const char* to_e,
                       const float* Ls, int s_e) __attribute__((always_inline)) {
      constexpr bool HS = decltype(hsc)::value, HE = decltype(hec)::value;
      bf16x8 pp[2];
      float lr = 0.f;  // LSE of part s_e, one row per lane (see stat_of)
      if (HE) lr = stat_load(Ls, s_e);
      const f32x16& xe = sv[s_e & 1];
      auto eslot = [&](int c) __attribute__((always_inline)) {
        bool used[2] = {false, false};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (pair_slot(j) != c) continue;
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int r = 2 * j + k;
            pp[r >> 3][r & 7] = (__bf16)fast_exp2(__builtin_fmaf(xe[r], sl, -stat_of(lr, r)));
          }
          used[j >> 2] = true;
        }
        // computed in this slot
        if (used[0]) asm volatile("" : "+v"(pp[0]));
        if (used[1]) asm volatile("" : "+v"(pp[1]));
      };
      if (HS)
        chain(tq, s, sv[s & 1], mask, qs, nullptr, [&](int c) {
          if (HE) eslot(c);
        });
      else if (HE) {
#pragma unroll
        for (int c = 0; c < DC; ++c) eslot(c);
      }
      if (HE) {
        char* pb = pbuf[grp][s_e & 1];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) *reinterpret_cast<bf16x8*>(pb + 1024 * mm + 16 * lane) = pp[mm];
        accumulate(to_e, s_e, pp);
      }
    };
    auto p_step = [&](int t, auto parity, auto firstc) {
      constexpr int par = decltype(parity)::value;
      constexpr bool FIRST = decltype(firstc)::value;
      const char* tq = par ? qbuf1 : qbuf0;
      const char* to = par ? obuf1 : obuf0;
      const int q0 = tile_start(t);
      const bool has_next = t + 1 < ntiles;
      const bool mask = tile_mask(q0);
#pragma unroll
      for (int s = 0; s < NH; ++s) {
        if (s == 2 && has_next) prefetch(t, std::integral_constant<int, par ^ 1>{});
        if (s > 0)
          p_phase(std::true_type{}, std::true_type{}, tq, s, mask, q0 + 32 * s, to, lbuf[par], s - 1);
        else if (!FIRST)
          p_phase(std::true_type{}, std::true_type{}, tq, s, mask, q0, par ? obuf0 : obuf1, lbuf[par ^ 1], NH - 1);
        else
          p_phase(std::true_type{}, std::false_type{}, tq, s, mask, q0, to, lbuf[par], 0);
        if (s == NH - 1) finish_tile(has_next, par ^ 1);
        lds_barrier();
      }
    };
    auto p_last = [&](auto parity) {  // parity of the last tile
      constexpr int par = decltype(parity)::value;
      p_phase(std::false_type{}, std::true_type{}, qbuf0, 0, false, 0, par ? obuf1 : obuf0, lbuf[par], NH - 1);
      lds_barrier();
    };
    if (ntiles > 0) {
      p_step(0, std::integral_constant<int, 0>{}, std::true_type{});
      for (int t = 1; t < ntiles; t += 2) {
        p_step(t, std::integral_constant<int, 1>{}, std::false_type{});
        if (t + 1 < ntiles) p_step(t + 1, std::integral_constant<int, 0>{}, std::false_type{});
      }
      if ((ntiles - 1) & 1)
        p_last(std::integral_constant<int, 1>{});
      else
        p_last(std::integral_constant<int, 0>{});
    }
  } else {
    f32x16 dpv[2];  // dP of part g in dpv[g & 1]
    // phase with dP of part s_p of buffers to_p (when HP) and dS / dK of part s_d of buffers
    // tq_d (when HD)
    auto ds_phase = [&](auto hpc, auto hdc, const char* to_p, int s_p, const char* tq_d, const float* Ds_d, int s_d)
        __attribute__((always_inline)) {
      constexpr bool HP = decltype(hpc)::value, HD = decltype(hdc)::value;
      bf16x8 pv[2], dsp[2];
      float dr = 0.f;  // D of part s_d, one row per lane (see stat_of)
      if (HD) {
        const char* pb = pbuf[grp][s_d & 1];
        pv[0] = lds_b128(pb + 16 * lane);
        pv[1] = lds_b128(pb + 1024 + 16 * lane);
        dr = stat_load(Ds_d, s_d);
#ifdef FA_CHECK
        // checking build: P consumed, its slots read as NaN until the P wave writes the next part
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(pv[0]), "+v"(pv[1]));
        lds_sentinel(const_cast<char*>(pb), 2, lane);
#endif
      }
      const f32x16& xd = dpv[s_d & 1];
      auto dslot = [&](int c) __attribute__((always_inline)) {
        bool used[2] = {false, false};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (pair_slot(j) != c) continue;
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int r = 2 * j + k;
            dsp[r >> 3][r & 7] = (__bf16)((float)pv[r >> 3][r & 7] * (xd[r] - stat_of(dr, r)));
          }
          used[j >> 2] = true;
        }
        // computed in this slot
        if (used[0]) asm volatile("" : "+v"(dsp[0]));
        if (used[1]) asm volatile("" : "+v"(dsp[1]));
      };
      if (HP)
        chain(to_p, s_p, dpv[s_p & 1], false, 0, nullptr, [&](int c) {
          if (HD) dslot(c);
        });
      else if (HD) {
#pragma unroll
        for (int c = 0; c < DC; ++c) dslot(c);
      }
      if (HD) accumulate(tq_d, s_d, dsp);
    };
    auto ds_step = [&](int t, auto parity, auto firstc) {
      constexpr int par = decltype(parity)::value;
      constexpr bool FIRST = decltype(firstc)::value;
      const char* tq = par ? qbuf1 : qbuf0;
      const char* to = par ? obuf1 : obuf0;
      const char* tq_prev = par ? qbuf0 : qbuf1;
      const char* to_prev = par ? obuf0 : obuf1;
      const bool has_next = t + 1 < ntiles;
#pragma unroll
      for (int s = 0; s < NH; ++s) {
        if (s == 2 && has_next) prefetch(t, std::integral_constant<int, par ^ 1>{});
        if (s >= 2)
          ds_phase(std::true_type{}, std::true_type{}, to, s - 1, tq, dbuf[par], s - 2);
        else if (s == 1) {
          if (FIRST)
            ds_phase(std::true_type{}, std::false_type{}, to, 0, tq, dbuf[par], 0);
          else
            ds_phase(std::true_type{}, std::true_type{}, to, 0, tq_prev, dbuf[par ^ 1], NH - 1);
        } else if (!FIRST) {
          ds_phase(std::true_type{}, std::true_type{}, to_prev, NH - 1, tq_prev, dbuf[par ^ 1], NH - 2);
        }
        if (s == NH - 1) finish_tile(has_next, par ^ 1);
        lds_barrier();
      }
    };
    auto ds_last = [&](auto parity) {  // parity of the last tile
      constexpr int par = decltype(parity)::value;
      const char* tq = par ? qbuf1 : qbuf0;
      const char* to = par ? obuf1 : obuf0;
      ds_phase(std::true_type{}, std::true_type{}, to, NH - 1, tq, dbuf[par], NH - 2);
      lds_barrier();
      ds_phase(std::false_type{}, std::true_type{}, to, 0, tq, dbuf[par], NH - 1);
    };
    if (ntiles > 0) {
      ds_step(0, std::integral_constant<int, 0>{}, std::true_type{});
      for (int t = 1; t < ntiles; t += 2) {
        ds_step(t, std::integral_constant<int, 1>{}, std::false_type{});
        if (t + 1 < ntiles) ds_step(t + 1, std::integral_constant<int, 0>{}, std::false_type{});
      }
      if ((ntiles - 1) & 1)
        ds_last(std::integral_constant<int, 1>{});
      else
        ds_last(std::integral_constant<int, 0>{});
    }
  }

  // ---- epilogue: lane holds feature 32 db + c32 of keys k0w + 8 g + 4 h + e (register 4 g + e)
  __bf16* __restrict__ dst = dsw ? a.dk : a.dv;
  const float f = dsw ? a.scale : 1.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = k0w + 8 * (r >> 2) + 4 * h + (r & 3);
      if (kr < N) dst[base + (size_t)kr * D + 32 * db + c32] = (__bf16)(acc[db][r] * f);
    }
}

// ------------------------------------------------------------------------------------------ dQ
template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a, Sched sc) {
  constexpr int BR = 128, BC = 64;
  constexpr int DC = D / 16, DB = D / 32;
  using KT = DmaTile<BC, D>;  // K (read row-wise and transposed) or V (row-wise)

  __shared__ __attribute__((aligned(1024))) char kbuf0[KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf1[KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf1[KT::BYTES];
  __shared__ unsigned short blist[SPARSE ? kMaxMaskBlocks : 1];
  __shared__ int bcount;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, c32 = lane & 31;
  const int N = a.N;
  int bh, qt;
  sched_decode(sc, gridDim.x, bh, qt);
  const int q0 = qt * BR;
  const size_t base = (size_t)bh * N * D;
  const size_t rbase = (size_t)bh * N;
  const __bf16* __restrict__ Kh = a.k + base;
  const __bf16* __restrict__ Vh = a.v + base;

  const int nk = (N + BC - 1) / BC;
  int ntiles = nk;
  if (CAUSAL) ntiles = min(nk, (min(q0 + BR, N) - 1) / BC + 1);
  if (SPARSE) {
    const int qb = q0 / kMaskBlock;
    if (w == 0) {
      const int cnt = build_block_list(a.mask, a.nb, qb, false, 0, CAUSAL ? qb + 1 : a.nb, blist, lane);
      if (lane == 0) bcount = cnt;
    }
    __syncthreads();
    const int cnt = bcount;
    ntiles = 2 * cnt;
    if (cnt > 0 && (int)blist[cnt - 1] * kMaskBlock + BC >= N) ntiles -= 1;
  }
  // causal query tiles of alternate cohorts walk the keys from the diagonal down
  // (sched_descending, as in the forward); the masks depend only on each tile's first key
  const bool desc = CAUSAL && !SPARSE && sched_descending(sc, gridDim.x);
  auto tile_start = [&](int t) -> int {
    if (SPARSE) return (int)blist[t >> 1] * kMaskBlock + (t & 1) * BC;
    return (desc ? ntiles - 1 - t : t) * BC;
  };

  const int qrow = q0 + 32 * w + c32;
  // Q (sign of the scale folded in) and dO rows in registers; rows past N load row N - 1 and are
  // zeroed, with no branch around the loads
  bf16x8 qreg[DC], doreg[DC];
  load_qt_operand(a.q + base, qrow, N, h, a.ssign, qreg);
  load_qt_operand(a.dout + base, qrow, N, h, 0u, doreg);
  float lse2 = __builtin_huge_valf(), dval = 0.f;
  if (qrow < N) {
    const float l = a.lse[rbase + qrow];
    lse2 = (l == neg_inf()) ? __builtin_huge_valf() : l * kLog2e;
    dval = a.delta[rbase + qrow];
  }
  f32x16 dqacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dqacc[i] = zero16();
  const float sl = a.scale_log2;

  // per-lane LDS addresses: A operands (K, V rows) and the transposed K^T reads
  int raddr[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) raddr[c] = KT::off(perm32(c32), 16 * c + 8 * h);
  int taddr[2][DB];
  {
    const int g = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) taddr[u][db] = KT::off4(8 * h + 4 * u + (j >> 2), 32 * db + 16 * g + 4 * (j & 3));
  }

  KT kdma, vdma;
  kdma.init(w, lane);
  vdma.init(w, lane);
  if (ntiles > 0) {
    kdma.issue(Kh, N, kbuf0, tile_start(0), w);
    vdma.issue(Vh, N, vbuf0, tile_start(0), w);
  }
  wait_dma();
  __syncthreads();

  // S^T = K Q^T and dP^T = V dO^T of key block kb of the tile: register r of half h holds key
  // k0 + 32 kb + acc_row(r, h), query qrow.  Operand reads run two MFMA pairs ahead; `hook(c)`
  // runs after MFMA pair c in the same fenced slot.  With `mask`, S^T starts at -inf on the
  // masked pairs (key >= N, or after the query when causal), so that P = 0 there.
  auto chain = [&](const char* tk, const char* tv, int kb, f32x16& sacc, f32x16& pacc, bool mask, int k0,
                   auto hook) __attribute__((always_inline)) {
    bf16x8 ka[DC], va[DC];
    auto rd = [&](int c) {
      ka[c] = lds_b128(tk + raddr[c] + 32 * kb * D * 2);
      va[c] = lds_b128(tv + raddr[c] + 32 * kb * D * 2);
    };
    rd(0);
    rd(1);
    if (mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = k0 + 32 * kb + acc_row(r, h);
        sacc[r] = (kr >= N || (CAUSAL && kr > qrow)) ? neg_inf() : 0.f;
      }
    } else {
      sacc = zero16();
    }
    pacc = zero16();
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      if (c + 2 < DC) rd(c + 2);
      __builtin_amdgcn_sched_barrier(0);
      sacc = mfma32(ka[c], qreg[c], sacc);
      pacc = mfma32(va[c], doreg[c], pacc);
      hook(c);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // slot c of `slots`: P = exp(S - LSE) and dS = P (dP - D) of 16 / slots score elements, as
  // bf16 B operands of dQ^T (dsp[m2] holds keys 16 m2 + 8h + 0..7 of the block)
  auto ds_slot = [&](const f32x16& sv, const f32x16& pv, bf16x8(&dsp)[2], int c, int slots)
      __attribute__((always_inline)) {
    const int per = 16 / slots, m2 = (per * c) >> 3;
#pragma unroll
    for (int k = 0; k < per; ++k) {
      const int r = per * c + k;
      const float p = fast_exp2(__builtin_fmaf(sv[r], sl, -lse2));
      dsp[m2][r & 7] = (__bf16)(p * (pv[r] - dval));
    }
    asm volatile("" : "+v"(dsp[m2]));  // computed in this slot
  };
  // dQ^T += K^T dS^T for key block kb (contraction over its 32 keys), K^T by transposing reads
  // kept two MFMAs ahead; `hook(i)` runs after MFMA i in the same fenced slot
  auto dq_mfmas = [&](const char* tk, int kb, const bf16x8(&dsp)[2], auto hook) __attribute__((always_inline)) {
    s16x4 tr[2 * DB][2];
    auto trd = [&](int i) {  // MFMA i: feature block i / 2, keys 16 (i % 2) ..
      const int roff = (32 * kb + 16 * (i & 1)) * D * 2;
      tr[i][0] = lds_tr4(tk + roff + taddr[0][i >> 1]);
      tr[i][1] = lds_tr4(tk + roff + taddr[1][i >> 1]);
    };
    trd(0);
    trd(1);
#pragma unroll
    for (int i = 0; i < 2 * DB; ++i) {
      if (i + 2 < 2 * DB) trd(i + 2);
      __builtin_amdgcn_sched_barrier(0);
      dqacc[i >> 1] = mfma32(join8(tr[i][0], tr[i][1]), dsp[i & 1], dqacc[i >> 1]);
      hook(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto step = [&](int t, auto parity) {
    constexpr int par = decltype(parity)::value;
    const char* tk = par ? kbuf1 : kbuf0;
    const char* tv = par ? vbuf1 : vbuf0;
    const int k0 = tile_start(t);
    const bool has_next = t + 1 < ntiles;
    if (has_next) {
      const int kn = tile_start(t + 1);
      kdma.issue(Kh, N, par ? kbuf0 : kbuf1, kn, w);
      vdma.issue(Vh, N, par ? vbuf0 : vbuf1, kn, w);
    }
    // tiles touching the key tail or the causal diagonal start S^T at -inf on masked pairs
    const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0 + 32 * w);
    // The two 32-key blocks of the tile, software-pipelined: the S^T / dP^T MFMAs of block 1
    // carry the exponentials and dS of block 0 in their slots, the dQ^T MFMAs of block 0 those
    // of block 1 (VALU work issued while the wave's own MFMAs run).
    f32x16 sa[2], pa[2];
    bf16x8 dsp[2][2];
    chain(tk, tv, 0, sa[0], pa[0], need_mask, k0, [](int) {});
    chain(tk, tv, 1, sa[1], pa[1], need_mask, k0, [&](int c) { ds_slot(sa[0], pa[0], dsp[0], c, DC); });
    dq_mfmas(tk, 0, dsp[0], [&](int i) { ds_slot(sa[1], pa[1], dsp[1], i, 2 * DB); });
    dq_mfmas(tk, 1, dsp[1], [](int) {});
    wait_dma();
    __syncthreads();
  };

  for (int t = 0; t < ntiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
  }

  if (qrow < N) {
    __bf16* row = a.dq + base + (size_t)qrow * D;
    const float scale = a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(dqacc[db][4 * g + e] * scale);
        *reinterpret_cast<bf16x4*>(row + 32 * db + 8 * g + 4 * h) = v4;
      }
  }
}

// ------------------------------------------------------------------ dK, dV and dQ in one pass
// The pre-pass of the one-pass backward: D per row (as bwd_delta_kernel) and zeros in the row's
// float32 dQ accumulator, which the one-pass kernel then adds into with atomics.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_zero_kernel(const __bf16* __restrict__ o,
                                                             const __bf16* __restrict__ dout, float* __restrict__ delta,
                                                             float* __restrict__ dq_acc, long rows) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const uint4 ov = *reinterpret_cast<const uint4*>(o + row * D + part * 8);
    const uint4 dv = *reinterpret_cast<const uint4*>(dout + row * D + part * 8);
    const __bf16* op = reinterpret_cast<const __bf16*>(&ov);
    const __bf16* dp = reinterpret_cast<const __bf16*>(&dv);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)op[e] * (float)dp[e];
    f32x4* z = reinterpret_cast<f32x4*>(dq_acc + row * D + part * 8);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    z[0] = zero;
    z[1] = zero;
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && part == 0) delta[row] = acc;
}

// dQ = scale * (float32 accumulator), rounded to bf16 (8 elements per thread)
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ dq_acc, __bf16* __restrict__ dq,
                                                             float scale, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = reinterpret_cast<const f32x4*>(dq_acc)[2 * i];
  const f32x4 b = reinterpret_cast<const f32x4*>(dq_acc)[2 * i + 1];
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (__bf16)(a[e] * scale);
    r[4 + e] = (__bf16)(b[e] * scale);
  }
  reinterpret_cast<bf16x8*>(dq)[i] = r;
}

// One pass over the query tiles of a 128-key block computing dV, dK and the block's share of dQ
// (d = 128).  Four waves, one per SIMD (512 registers each): wave w owns keys k0 + 32 w .. + 31
// and, for dQ, features 32 w .. + 31.  Per 32-query part of a query tile:
//   S = Q K^T, dP = dO V^T         (K, V rows of the wave's keys in registers, Q / dO rows from LDS)
//   P = exp(S - LSE), dS = P (dP - D)
//   dV += P^T dO, dK += dS^T Q
//   dS (bf16) to LDS; after the part barrier every wave reads the dS of all 128 keys (transposed)
//   and computes dQ[part, its 32 features] = dS K over the block, K^T read transposed from the
//   block's K rows kept in LDS, then adds it with float32 atomics into the caller's accumulator.
// Each dQ element gets one atomic add per key block, so the atomics move exactly the bytes of the
// dQ partials.  The dQ of a part runs in the step of the next part, and its MFMAs carry that part's
// exponentials in their slots (the dV MFMAs carry dS), so one part's S and dP are live at a time.
// Query tiles are 64 rows (two parts), double-buffered: with the K block (32 KB) and the dS
// exchange (16 KB) LDS holds 114 KB.  S, P, dP and dS are the values bwd_dkdv_wave_kernel computes.
template <bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 1) void bwd_fused_kernel(BwdArgs a, Sched sc, float* __restrict__ dq_acc) {
  constexpr int D = 128, BKV = 128, BQ = 64;
  constexpr int NH = BQ / 32;
  constexpr int DC = D / 16, DB = D / 32;
  using QT = DmaTile<BQ, D>;   // Q or dO rows of a query tile
  using KB = DmaTile<BKV, D>;  // the key block's K rows

  __shared__ __attribute__((aligned(1024))) char qbuf0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char qbuf1[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char obuf0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char obuf1[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char kblk[KB::BYTES];
  __shared__ __attribute__((aligned(1024))) char dsbuf[2][4][2048];  // dS of a part: [parity][key group][key][query]
  __shared__ __attribute__((aligned(16))) float lbuf[2][BQ];
  __shared__ __attribute__((aligned(16))) float dbuf[2][BQ];
  __shared__ unsigned short blist[SPARSE ? kMaxMaskBlocks : 1];
  __shared__ int bcount;

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5,
            c32 = lane & 31;
  const int N = a.N;
  int bh, kt;
  sched_decode(sc, gridDim.x, bh, kt);
  const int k0 = kt * BKV;
  const int k0w = k0 + 32 * w;
  const size_t base = (size_t)bh * N * D;
  const size_t rbase = (size_t)bh * N;
  const __bf16* __restrict__ Qh = a.q + base;
  const __bf16* __restrict__ Oh = a.dout + base;

  // ---- query tiles (64 rows, two per 128-row mask block) that see this key block
  const int nqt = (N + BQ - 1) / BQ;
  int q_first = 0, ntiles = nqt;
  if (CAUSAL) {
    q_first = k0 / BQ;
    ntiles = nqt - q_first;
  }
  if (SPARSE) {
    if (w == 0) {
      const int cnt = build_block_list(a.mask, a.nb, kt, true, CAUSAL ? kt : 0, a.nb, blist, lane);
      if (lane == 0) bcount = cnt;
    }
    __syncthreads();
    const int cnt = bcount;
    ntiles = 2 * cnt;
    if (cnt > 0 && (int)blist[cnt - 1] * kMaskBlock + BQ >= N) ntiles -= 1;  // last block's second half past N
  }
  auto tile_start = [&](int t) -> int {
    if (SPARSE) return (int)blist[t >> 1] * kMaskBlock + (t & 1) * BQ;
    return (q_first + t) * BQ;
  };

  // ---- this lane's key: K (sign of scale folded in) and V rows as the B operands of S and dP
  const int key = k0w + c32;
  bf16x8 kreg[DC], vreg[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    if (key < N) {
      kreg[c] = xor_sign(*reinterpret_cast<const bf16x8*>(a.k + base + (size_t)key * D + 16 * c + 8 * h), a.ssign);
      vreg[c] = *reinterpret_cast<const bf16x8*>(a.v + base + (size_t)key * D + 16 * c + 8 * h);
    } else {
      kreg[c] = zero_bf16x8();
      vreg[c] = zero_bf16x8();
    }
  }
  f32x16 dvacc[DB], dkacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dvacc[i] = zero16();
    dkacc[i] = zero16();
  }
  const float sl = a.scale_log2;

  int raddr[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) raddr[c] = QT::off(perm32(c32), 16 * c + 8 * h);
  int taddr[2][DB];
  {
    const int g = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db) taddr[u][db] = QT::off4(8 * h + 4 * u + (j >> 2), 32 * db + 16 * g + 4 * (j & 3));
  }
  // transposed read u of a 16-key chunk of dS (rows = keys, 32 queries per 64-byte row): lane j
  // of its 16-lane group addresses key row 8h + 4u + j/4 (+ 16 (chunk % 2)), queries 16g + 4(j % 4);
  // and of K^T: key row 8h + 4u + j/4 (+ 16 chunk), features 32 w + 16g + 4(j % 4)
  int daddr[2], kaddr[2];
  {
    const int g = (lane >> 4) & 1, j = lane & 15;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      daddr[u] = (8 * h + 4 * u + (j >> 2)) * 64 + (16 * g + 4 * (j & 3)) * 2;
      kaddr[u] = KB::off4(8 * h + 4 * u + (j >> 2), 32 * w + 16 * g + 4 * (j & 3));
    }
  }

  QT qdma, odma;
  qdma.init(w, lane);
  odma.init(w, lane);
  float lpre = 0.f, dlpre = 0.f;
  auto rowstats_load = [&](int q0) {
    if (tid < BQ) {
      const int qr = q0 + tid;
      const float l = qr < N ? a.lse[rbase + qr] : neg_inf();
      lpre = (l == neg_inf()) ? __builtin_huge_valf() : l * kLog2e;
      dlpre = qr < N ? a.delta[rbase + qr] : 0.f;
    }
  };
  auto rowstats_store = [&](int buf) {
    if (tid < BQ) {
      lbuf[buf][tid] = lpre;
      dbuf[buf][tid] = dlpre;
    }
  };

  {
    KB kdma;
    kdma.init(w, lane);
    kdma.issue(a.k + base, N, kblk, k0, w);
  }
  if (ntiles > 0) {
    const int q0 = tile_start(0);
    qdma.issue(Qh, N, qbuf0, q0, w);
    odma.issue(Oh, N, obuf0, q0, w);
    rowstats_load(q0);
    wait_dma();
    rowstats_store(0);
  }
  wait_dma();
  __syncthreads();

  // S = Q K^T and dP = dO V^T of part s: register r of half h holds query 32 s + acc_row(r, h) of
  // the tile, key `key`; operand reads two MFMA pairs ahead; S starts at -inf on masked pairs
  // (the key tail, and the causal diagonal for the part's queries qs ..).  Compiler MFMAs: the
  // compiler places the accumulators and inserts the wait states around them.
  auto sp_chain = [&](const char* tq, const char* to, int s, f32x16& sacc, f32x16& pacc, bool mask, int qs)
      __attribute__((always_inline)) {
    bf16x8 qa[DC], oa[DC];
    auto rd = [&](int c) {
      qa[c] = lds_b128(tq + raddr[c] + 32 * s * D * 2);
      oa[c] = lds_b128(to + raddr[c] + 32 * s * D * 2);
    };
    rd(0);
    rd(1);
    if (mask) {
      const int thr = key >= N ? 32 : (CAUSAL ? key - qs - 8 * h : 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 16 * (r >> 3) + (r & 7) < thr ? neg_inf() : 0.f;
    } else {
      sacc = zero16();
    }
    pacc = zero16();
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      if (c + 2 < DC) rd(c + 2);
      __builtin_amdgcn_sched_barrier(0);
      sacc = mfma32(qa[c], kreg[c], sacc);
      pacc = mfma32(oa[c], vreg[c], pacc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto stat4 = [&](const float* rows, int s, int qq) -> f32x4 {
    return *reinterpret_cast<const f32x4*>(rows + 32 * s + 16 * (qq >> 1) + 8 * h + 4 * (qq & 1));
  };
  auto p_quarter = [&](f32x16& x, const f32x4& l, int qq, bf16x8(&pp)[2]) __attribute__((always_inline)) {
    const int mm = qq >> 1, e0 = 4 * (qq & 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 8 * mm + e0 + e;
      const float p = fast_exp2(__builtin_fmaf(x[r], sl, -l[e]));
      x[r] = p;
      pp[mm][e0 + e] = (__bf16)p;
    }
  };
  auto ds_quarter = [&](const f32x16& x, const f32x16& y, const f32x4& d, int qq, bf16x8(&dsp)[2])
      __attribute__((always_inline)) {
    const int mm = qq >> 1, e0 = 4 * (qq & 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 8 * mm + e0 + e;
      dsp[mm][e0 + e] = (__bf16)(x[r] * (y[r] - d[e]));
    }
  };
  auto acc_mfma = [](f32x16& acc, const bf16x8& x, const bf16x8& y) __attribute__((always_inline)) {
    acc = mfma32(x, y, acc);
  };
  auto dvdk = [&](const char* tq, const char* to, int s, const bf16x8(&pp)[2], const f32x16& x, const f32x16& y,
                  const float* Ds, bf16x8(&dsp)[2]) __attribute__((always_inline)) {
    bf16x8 ob[2 * DB], qb[2 * DB];
    auto trd = [&](const char* t, int i) -> bf16x8 {
      const int db = i >> 1, roff = (32 * s + 16 * (i & 1)) * D * 2;
      return join8(lds_tr4(t + roff + taddr[0][db]), lds_tr4(t + roff + taddr[1][db]));
    };
    ob[0] = trd(to, 0);
    ob[1] = trd(to, 1);
    f32x4 d = stat4(Ds, s, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * DB; ++i) {
      if (i + 2 < 2 * DB) ob[i + 2] = trd(to, i + 2);
      else qb[i + 2 - 2 * DB] = trd(tq, i + 2 - 2 * DB);
      acc_mfma(dvacc[i >> 1], pp[i & 1], ob[i]);
      if (i & 1) {
        const int qq = i >> 1;
        const f32x4 dc = d;
        if (qq + 1 < 4) d = stat4(Ds, s, qq + 1);
        ds_quarter(x, y, dc, qq, dsp);
        if (qq & 1) asm volatile("" : "+v"(dsp[qq >> 1]));  // computed in this slot
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 2 * DB; ++i) {
      if (i + 2 < 2 * DB) qb[i + 2] = trd(tq, i + 2);
      acc_mfma(dkacc[i >> 1], dsp[i & 1], qb[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // dQ of the part whose dS is in dsbuf[par] (queries qs ..): 8 MFMAs over the block's 128 keys
  // (dS and K^T read transposed), then 16 float32 atomic adds of the wave's 32 features: register
  // r of half h holds query qs + 8 (r / 4) + 4h + r % 4, feature 32 w + c32.  The adds go through a
  // buffer resource that starts at row qs and ends at row N: the per-lane offsets are fixed (rows
  // 8 (r / 4) + 4h, the r % 4 part in the instruction's offset), and the hardware range check drops
  // the adds of rows past N.  Every add is issued, so the count per step is fixed.
  int avo[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) avo[m] = ((8 * m + 4 * h) * D + 32 * w + c32) * 4;
  auto dq_part = [&](int par, int qs, auto hook) __attribute__((always_inline)) {
    f32x16 acc;
    bf16x8 dsa[8], kta[8];
    auto rd = [&](int j) {
      const char* src = &dsbuf[par][j >> 1][0] + 16 * (j & 1) * 64;
      dsa[j] = join8(lds_tr4(src + daddr[0]), lds_tr4(src + daddr[1]));
      const char* ksrc = kblk + 16 * j * D * 2;
      kta[j] = join8(lds_tr4(ksrc + kaddr[0]), lds_tr4(ksrc + kaddr[1]));
    };
    rd(0);
    rd(1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j + 2 < 8) rd(j + 2);
      __builtin_amdgcn_sched_barrier(0);
      acc = mfma32(dsa[j], kta[j], j == 0 ? zero16() : acc);
      hook(j);
      __builtin_amdgcn_sched_barrier(0);
    }
    const Rsrc rs = make_rsrc(dq_acc + (rbase + qs) * D, max(N - qs, 0) * D * 4);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r], rs, avo[r >> 2] + (r & 3) * D * 4, 0, 0);
  };

  auto step = [&](int t, auto parity) {
    constexpr int par = decltype(parity)::value;
    const char* tq = par ? qbuf1 : qbuf0;
    const char* to = par ? obuf1 : obuf0;
    const int q0 = tile_start(t);
    const bool has_next = t + 1 < ntiles;
    if (has_next) {
      const int qn = tile_start(t + 1);
      qdma.issue(Qh, N, par ? qbuf0 : qbuf1, qn, w);
      odma.issue(Oh, N, par ? obuf0 : obuf1, qn, w);
      rowstats_load(qn);
    }
    const float* Ls = lbuf[par];
    const float* Ds = dbuf[par];
    auto part_mask = [&](int qs) -> bool { return (k0w + 32 > N) || (CAUSAL && qs < k0w + 31); };
    // Part s of the tile: the S / dP MFMAs; then the previous part's dQ MFMAs with this part's
    // exponentials in their slots (a quarter of P per two MFMAs, the LSE read one quarter ahead)
    // and its atomic adds; then dV (dS in its slots) and dK; dS to LDS; the part barrier.
#pragma unroll
    for (int s = 0; s < NH; ++s) {
      const int qs = q0 + 32 * s;
      f32x16 x, y;  // S (then P in fp32) and dP of the part
      bf16x8 pp[2], dsp[2];
      sp_chain(tq, to, s, x, y, part_mask(qs), qs);
      f32x4 l = stat4(Ls, s, 0);
      auto quarter = [&](int qq) __attribute__((always_inline)) {
        const f32x4 lc = l;
        if (qq + 1 < 4) l = stat4(Ls, s, qq + 1);
        p_quarter(x, lc, qq, pp);
        if (qq & 1) asm volatile("" : "+v"(pp[qq >> 1]));  // computed in this slot
      };
      auto quarter_slot = [&](int j) __attribute__((always_inline)) {
        if (j & 1) quarter(j >> 1);
      };
      if (s > 0)
        dq_part(0, q0, quarter_slot);
      else if (t > 0)
        dq_part(1, tile_start(t - 1) + 32, quarter_slot);
      else {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) quarter(qq);
      }
      dvdk(tq, to, s, pp, x, y, Ds, dsp);
      // dS of this part (global part 2t + s, parity s) to LDS: key c32 of the group, queries
      // 16 mm + 8h ..
      char* dsw = &dsbuf[s][w][0] + c32 * 64 + 16 * h;
      *reinterpret_cast<bf16x8*>(dsw) = dsp[0];
      *reinterpret_cast<bf16x8*>(dsw + 32) = dsp[1];
      if (s == NH - 1) {
        if (has_next) rowstats_store(par ^ 1);
        // the next tile's copies were issued before this tile's atomic adds (16 per dQ part)
        if (t > 0)
          wait_vm<32>();
        else
          wait_vm<16>();
      }
      lds_barrier();
    }
  };

  for (int t = 0; t < ntiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
  }
  if (ntiles > 0) dq_part(1, tile_start(ntiles - 1) + 32, [](int) {});  // the last part's dQ

  // ---- epilogue: lane holds feature 32 db + c32 of keys k0w + 8 g + 4 h + e (register 4 g + e)
  const float scale = a.scale;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = k0w + 8 * (r >> 2) + 4 * h + (r & 3);
      if (kr < N) {
        const size_t off = base + (size_t)kr * D + 32 * db + c32;
        a.dv[off] = (__bf16)dvacc[db][r];
        a.dk[off] = (__bf16)(dkacc[db][r] * scale);
      }
    }
}

template <int D>
hipError_t launch_delta_t(const BwdArgs& a, hipStream_t st) {
  const long rows = (long)a.BH * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_delta_kernel<__bf16, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, a.o,
                     a.dout, a.delta, rows);
  return hipGetLastError();
}

template <int D, bool C, bool S>
hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t st) {
  const int nkv = (a.N + 127) / 128;
  if constexpr (D == 64) {
    static const int slots = xcd_slots(reinterpret_cast<const void*>(&bwd_dkdv_wave_kernel<D, C, S>), 256);
    const Sched sc = make_sched(nkv, a.BH, /*heavy_last_tile=*/0, slots, /*uneven=*/C || S);
    hipLaunchKernelGGL((bwd_dkdv_wave_kernel<D, C, S>), dim3(nkv * a.BH), dim3(256), 0, st, a, sc);
  } else {
    static const int slots = xcd_slots(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, C, S>), 512);
    const Sched sc = make_sched(nkv, a.BH, /*heavy_last_tile=*/0, slots, /*uneven=*/C || S);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, C, S>), dim3(nkv * a.BH), dim3(512), 0, st, a, sc);
  }
  return hipGetLastError();
}

template <int D, bool C, bool S>
hipError_t launch_dq_t(const BwdArgs& a, hipStream_t st) {
  const int nq = (a.N + 127) / 128;
  static const int slots = xcd_slots(reinterpret_cast<const void*>(&bwd_dq_kernel<D, C, S>));
  const Sched sc = make_sched(nq, a.BH, /*heavy_last_tile=*/1, slots, /*uneven=*/C || S, /*alternate=*/C && !S);
  hipLaunchKernelGGL((bwd_dq_kernel<D, C, S>), dim3(nq * a.BH), dim3(256), 0, st, a, sc);
  return hipGetLastError();
}

// dispatch on (d, causal, sparse) to a kernel template instantiation
template <template <int, bool, bool> class L>
hipError_t dispatch(const BwdArgs& a, hipStream_t st) {
  const bool c = a.causal != 0, s = a.mask != nullptr;
  if (a.d == 64) {
    if (c) return s ? L<64, true, true>::run(a, st) : L<64, true, false>::run(a, st);
    return s ? L<64, false, true>::run(a, st) : L<64, false, false>::run(a, st);
  }
  if (c) return s ? L<128, true, true>::run(a, st) : L<128, true, false>::run(a, st);
  return s ? L<128, false, true>::run(a, st) : L<128, false, false>::run(a, st);
}

template <int D, bool C, bool S>
struct DkdvL {
  static hipError_t run(const BwdArgs& a, hipStream_t st) { return launch_dkdv_t<D, C, S>(a, st); }
};
template <int D, bool C, bool S>
struct DqL {
  static hipError_t run(const BwdArgs& a, hipStream_t st) { return launch_dq_t<D, C, S>(a, st); }
};

template <bool C, bool S>
hipError_t launch_fused_t(const BwdArgs& a, float* dq_acc, hipStream_t st) {
  const int nkv = (a.N + 127) / 128;
  static const int slots = xcd_slots(reinterpret_cast<const void*>(&bwd_fused_kernel<C, S>), 256);
  const Sched sc = make_sched(nkv, a.BH, /*heavy_last_tile=*/0, slots, /*uneven=*/C || S);
  hipLaunchKernelGGL((bwd_fused_kernel<C, S>), dim3(nkv * a.BH), dim3(256), 0, st, a, sc, dq_acc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prepass_zero_bf16(const BwdArgs& a, float* dq_acc, hipStream_t st) {
  const long rows = (long)a.BH * a.N;
  constexpr int RPB = 256 / (128 / 8);
  hipLaunchKernelGGL((bwd_delta_zero_kernel<128>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, a.o,
                     a.dout, a.delta, dq_acc, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdvq_bf16(const BwdArgs& a, float* dq_acc, hipStream_t st) {
  const bool c = a.causal != 0, s = a.mask != nullptr;
  if (c) return s ? launch_fused_t<true, true>(a, dq_acc, st) : launch_fused_t<true, false>(a, dq_acc, st);
  return s ? launch_fused_t<false, true>(a, dq_acc, st) : launch_fused_t<false, false>(a, dq_acc, st);
}

hipError_t launch_bwd_dq_convert_bf16(const BwdArgs& a, const float* dq_acc, hipStream_t st) {
  const long n8 = (long)a.BH * a.N * a.d / 8;
  hipLaunchKernelGGL(bwd_dq_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, dq_acc, a.dq, a.scale,
                     n8);
  return hipGetLastError();
}

hipError_t launch_bwd_onepass_bf16(const BwdArgs& a, float* dq_acc, hipStream_t stream) {
  hipError_t e = launch_bwd_prepass_zero_bf16(a, dq_acc, stream);
  if (e != hipSuccess) return e;
  e = launch_bwd_dkdvq_bf16(a, dq_acc, stream);
  if (e != hipSuccess) return e;
  return launch_bwd_dq_convert_bf16(a, dq_acc, stream);
}

hipError_t launch_bwd_delta_bf16(const BwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch_delta_t<64>(a, stream) : launch_delta_t<128>(a, stream);
}

hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, hipStream_t stream) { return dispatch<DkdvL>(a, stream); }

hipError_t launch_bwd_dq_bf16(const BwdArgs& a, hipStream_t stream) { return dispatch<DqL>(a, stream); }

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  hipError_t e = launch_bwd_delta_bf16(a, stream);
  if (e != hipSuccess) return e;
  e = launch_bwd_dkdv_bf16(a, stream);
  if (e != hipSuccess) return e;
  return launch_bwd_dq_bf16(a, stream);
}

// The fp32 path shares the D pre-pass kernel.
hipError_t launch_delta_f32(const float* o, const float* dout, float* delta, long rows, int d, hipStream_t st) {
  if (d == 64) {
    constexpr int RPB = 256 / (64 / 4);
    hipLaunchKernelGGL((bwd_delta_kernel<float, 64>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, o,
                       dout, delta, rows);
  } else {
    constexpr int RPB = 256 / (128 / 4);
    hipLaunchKernelGGL((bwd_delta_kernel<float, 128>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, o,
                       dout, delta, rows);
  }
  return hipGetLastError();
}

}  // namespace fa
