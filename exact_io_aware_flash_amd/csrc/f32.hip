// float32 path: the same tiled forward with online softmax and the same recompute backward,
// with every product and sum in fp32 (no reduced-precision matrix instructions).  It serves
// fp32 callers that need errors near fp32 rounding; the bf16 MFMA kernels are the fast path.
//
// Layout: each query (or key) row is owned by G = d / 32 adjacent lanes, each holding 32 of the
// d columns in registers; dot products are reduced across the G lanes with shuffles.  K/V (or
// Q/dO) tiles of 32 rows are staged in LDS, where every lane of a row group reads the same row
// (broadcast).  Visibility (key tail, causal, 128 x 128 block mask) is applied per element.
//
// Method: [P2] "FlashAttention: how a memory trick unlocked today's giant AI models", sections
// "Tiling: Breaking the Problem into Pieces" and "The Trick: Online Softmax"; backward from the
// saved row statistic, [P3] "How FlashAttention Eliminates Transformer Memory Bottlenecks",
// "Innovation #3".
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

hipError_t launch_delta_f32(const float* o, const float* dout, float* delta, long rows, int d, hipStream_t st);

namespace {

constexpr int TR = 32;  // rows per LDS tile

template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ bool visible(int qi, int kj, int N, bool causal, const uint8_t* mask, int nb) {
  if (kj >= N || qi >= N) return false;
  if (causal && kj > qi) return false;
  if (mask && mask[(size_t)(qi / kMaskBlock) * nb + (kj / kMaskBlock)] == 0) return false;
  return true;
}

template <int D>
__device__ __forceinline__ void load_tile(float (*dst)[D], const float* src, int r0, int N) {
  // TR x D floats, 16-byte loads, rows past N zero-filled
  for (int i = threadIdx.x; i < TR * D / 4; i += 256) {
    const int row = i / (D / 4), col = (i % (D / 4)) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r0 + row < N) v = *reinterpret_cast<const float4*>(src + (size_t)(r0 + row) * D + col);
    *reinterpret_cast<float4*>(&dst[row][col]) = v;
  }
}

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(F32Args a) {
  constexpr int G = D / 32, RPB = 256 / G;
  __shared__ __attribute__((aligned(16))) float ks[TR][D];
  __shared__ __attribute__((aligned(16))) float vs[TR][D];
  const int N = a.N, bh = blockIdx.y;
  const int sub = threadIdx.x % G;
  const int qi = blockIdx.x * RPB + threadIdx.x / G;
  const size_t base = (size_t)bh * N * D;
  const bool causal = a.causal != 0;
  float qv[32], ov[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    qv[c] = qi < N ? a.q[base + (size_t)qi * D + 32 * sub + c] : 0.f;
    ov[c] = 0.f;
  }
  float m = neg_inf(), l = 0.f;
  const int kend = causal ? min(N, (blockIdx.x + 1) * RPB) : N;
  for (int k0 = 0; k0 < kend; k0 += TR) {
    __syncthreads();
    load_tile<D>(ks, a.k + base, k0, N);
    load_tile<D>(vs, a.v + base, k0, N);
    __syncthreads();
    float s[TR];
    float mt = neg_inf();
#pragma unroll
    for (int j = 0; j < TR; ++j) {
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < 32; ++c) part = __builtin_fmaf(qv[c], ks[j][32 * sub + c], part);
      const float full = group_sum<G>(part) * a.scale;
      s[j] = visible(qi, k0 + j, N, causal, a.mask, a.nb) ? full : neg_inf();
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m, mt);
    if (m_new != neg_inf()) {
      const float alpha = (m == neg_inf()) ? 0.f : expf(m - m_new);
#pragma unroll
      for (int c = 0; c < 32; ++c) ov[c] *= alpha;
      l *= alpha;
#pragma unroll
      for (int j = 0; j < TR; ++j) {
        const float p = (s[j] == neg_inf()) ? 0.f : expf(s[j] - m_new);
        l += p;
#pragma unroll
        for (int c = 0; c < 32; ++c) ov[c] = __builtin_fmaf(p, vs[j][32 * sub + c], ov[c]);
      }
      m = m_new;
    }
  }
  if (qi < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) a.out_o[base + (size_t)qi * D + 32 * sub + c] = ov[c] * inv;
    if (sub == 0) a.lse[(size_t)bh * N + qi] = l > 0.f ? m + logf(l) : neg_inf();
  }
}

template <int D>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(F32Args a) {
  constexpr int G = D / 32, RPB = 256 / G;
  __shared__ __attribute__((aligned(16))) float qs[TR][D];
  __shared__ __attribute__((aligned(16))) float dos[TR][D];
  __shared__ float ls[TR], dl[TR];
  const int N = a.N, bh = blockIdx.y;
  const int sub = threadIdx.x % G;
  const int kj = blockIdx.x * RPB + threadIdx.x / G;
  const size_t base = (size_t)bh * N * D, rbase = (size_t)bh * N;
  const bool causal = a.causal != 0;
  float kv[32], vv[32], dk[32], dv[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    kv[c] = kj < N ? a.k[base + (size_t)kj * D + 32 * sub + c] : 0.f;
    vv[c] = kj < N ? a.v[base + (size_t)kj * D + 32 * sub + c] : 0.f;
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  const int qstart = causal ? (blockIdx.x * RPB / TR) * TR : 0;
  for (int q0 = qstart; q0 < N; q0 += TR) {
    __syncthreads();
    load_tile<D>(qs, a.q + base, q0, N);
    load_tile<D>(dos, a.dout + base, q0, N);
    if (threadIdx.x < TR) {
      const int qi = q0 + threadIdx.x;
      ls[threadIdx.x] = qi < N ? a.lse[rbase + qi] : 0.f;
      dl[threadIdx.x] = qi < N ? a.delta[rbase + qi] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int i = 0; i < TR; ++i) {
      float ps = 0.f, pd = 0.f;
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        ps = __builtin_fmaf(kv[c], qs[i][32 * sub + c], ps);
        pd = __builtin_fmaf(vv[c], dos[i][32 * sub + c], pd);
      }
      const float s = group_sum<G>(ps) * a.scale;
      const float dp = group_sum<G>(pd);
      const float p = visible(q0 + i, kj, N, causal, a.mask, a.nb) ? expf(s - ls[i]) : 0.f;
      const float ds = p * (dp - dl[i]);
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        dv[c] = __builtin_fmaf(p, dos[i][32 * sub + c], dv[c]);
        dk[c] = __builtin_fmaf(ds, qs[i][32 * sub + c], dk[c]);
      }
    }
  }
  if (kj < N) {
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      a.dk[base + (size_t)kj * D + 32 * sub + c] = dk[c] * a.scale;
      a.dv[base + (size_t)kj * D + 32 * sub + c] = dv[c];
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void dq_f32_kernel(F32Args a) {
  constexpr int G = D / 32, RPB = 256 / G;
  __shared__ __attribute__((aligned(16))) float ks[TR][D];
  __shared__ __attribute__((aligned(16))) float vs[TR][D];
  const int N = a.N, bh = blockIdx.y;
  const int sub = threadIdx.x % G;
  const int qi = blockIdx.x * RPB + threadIdx.x / G;
  const size_t base = (size_t)bh * N * D, rbase = (size_t)bh * N;
  const bool causal = a.causal != 0;
  float qv[32], dov[32], dq[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    qv[c] = qi < N ? a.q[base + (size_t)qi * D + 32 * sub + c] : 0.f;
    dov[c] = qi < N ? a.dout[base + (size_t)qi * D + 32 * sub + c] : 0.f;
    dq[c] = 0.f;
  }
  const float lse = qi < N ? a.lse[rbase + qi] : 0.f;
  const float dl = qi < N ? a.delta[rbase + qi] : 0.f;
  const int kend = causal ? min(N, (blockIdx.x + 1) * RPB) : N;
  for (int k0 = 0; k0 < kend; k0 += TR) {
    __syncthreads();
    load_tile<D>(ks, a.k + base, k0, N);
    load_tile<D>(vs, a.v + base, k0, N);
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < TR; ++j) {
      float ps = 0.f, pd = 0.f;
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        ps = __builtin_fmaf(qv[c], ks[j][32 * sub + c], ps);
        pd = __builtin_fmaf(dov[c], vs[j][32 * sub + c], pd);
      }
      const float s = group_sum<G>(ps) * a.scale;
      const float dp = group_sum<G>(pd);
      const float p = visible(qi, k0 + j, N, causal, a.mask, a.nb) ? expf(s - lse) : 0.f;
      const float ds = p * (dp - dl);
#pragma unroll
      for (int c = 0; c < 32; ++c) dq[c] = __builtin_fmaf(ds, ks[j][32 * sub + c], dq[c]);
    }
  }
  if (qi < N) {
#pragma unroll
    for (int c = 0; c < 32; ++c) a.dq[base + (size_t)qi * D + 32 * sub + c] = dq[c] * a.scale;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const F32Args& a, hipStream_t st) {
  const int RPB = 256 / (a.d / 32);
  const dim3 grid((a.N + RPB - 1) / RPB, a.BH);
  if (a.d == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const F32Args& a, hipStream_t st) {
  hipError_t e = launch_delta_f32(a.o, a.dout, a.delta, (long)a.BH * a.N, a.d, st);
  if (e != hipSuccess) return e;
  const int RPB = 256 / (a.d / 32);
  const dim3 grid((a.N + RPB - 1) / RPB, a.BH);
  if (a.d == 64) {
    hipLaunchKernelGGL(dkdv_f32_kernel<64>, grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL(dq_f32_kernel<64>, grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(dkdv_f32_kernel<128>, grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL(dq_f32_kernel<128>, grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace fa
