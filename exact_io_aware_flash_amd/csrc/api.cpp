// C ABI of the attention library: argument validation on the host, then kernel launches.
// Every check runs before the first HIP call, so an invalid call enqueues nothing and touches
// no output (and can be exercised on a machine without a GPU).
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/flash_attn.h"
#include "fa_kernels.h"

namespace {

constexpr long long kMaxElems = (1LL << 62);
static_assert(FA_NOALLOC_MAX_ROWS == fa::kNoallocMaxRows, "header and library agree on the fixed scratch");

struct Range {
  uintptr_t lo, hi;
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int B, int H, int N, int d, float scale, int causal, const uint8_t* block_mask, bool bf16,
                 long long* elems) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (!std::isfinite(scale) || scale == 0.f) return FA_ERR_SCALE;
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  // one head's slice must be a 31-bit byte range (checked first: it bounds N * d to 2^29, so
  // the products below stay far inside 64 bits)
  if ((long long)N * d * 4 > 0x7fffffffLL) return FA_ERR_SHAPE;
  const long long bh = (long long)B * H;
  if (bh > (1LL << 30)) return FA_ERR_SHAPE;
  const long long e = bh * ((long long)N * d);
  if (e <= 0 || e >= kMaxElems / 4) return FA_ERR_SHAPE;
  const long long nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  if (block_mask && bf16 && nb > FA_MAX_MASK_BLOCKS) return FA_ERR_SHAPE;
  if (!bf16 && bh > 65535) return FA_ERR_SHAPE;  // the fp32 kernels put B*H on grid.y
  const long long tiles = bh * ((N + 127) / 128);
  if (tiles > 0x7fffffffLL) return FA_ERR_SHAPE;
  *elems = e;
  return FA_OK;
}

Range rng(const void* p, long long bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)bytes};
}

// outputs must not overlap inputs or each other
int check_alias(const Range* in, int nin, const Range* out, int nout) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(out[i], in[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(out[i], out[j])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

size_t workspace_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return fa::ws_bytes((long long)B * H, N);
}

template <typename T>
int fwd_checked(const T* q, const T* k, const T* v, T* o, float* lse, int B, int H, int N, int d, float scale,
                int causal, const uint8_t* block_mask, bool bf16, long long* elems) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal, block_mask, bf16, elems);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  const long long tb = *elems * (long long)sizeof(T), lb = (long long)B * H * N * 4;
  const long long nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  Range in[4] = {rng(q, tb), rng(k, tb), rng(v, tb), rng(block_mask, block_mask ? nb * nb : 0)};
  Range out[2] = {rng(o, tb), rng(lse, lb)};
  return check_alias(in, 4, out, 2);
}

template <typename T>
int bwd_checked(const T* q, const T* k, const T* v, const T* o, const T* dout, const float* lse, T* dq, T* dk, T* dv,
                void* ws, size_t ws_bytes, int B, int H, int N, int d, float scale, int causal,
                const uint8_t* block_mask, bool bf16, long long* elems) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale, causal, block_mask, bf16, elems);
  if (st != FA_OK) return st;
  if (!ws || ws_bytes < workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  const long long tb = *elems * (long long)sizeof(T), lb = (long long)B * H * N * 4;
  const long long nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  Range in[7] = {rng(q, tb),    rng(k, tb),   rng(v, tb), rng(o, tb), rng(dout, tb), rng(lse, lb),
                 rng(block_mask, block_mask ? nb * nb : 0)};
  Range out[4] = {rng(dq, tb), rng(dk, tb), rng(dv, tb), rng(ws, (long long)workspace_bytes(B, H, N, d))};
  return check_alias(in, 7, out, 4);
}

// Shared checks for the bf16 backward stages: all pointers non-null and aligned, shapes and
// flags valid, outputs disjoint from inputs and from each other.
int stage_checked(const void* const* in, const long long* in_bytes, int nin, void* const* out,
                  const long long* out_bytes, int nout, int B, int H, int N, int d, float scale, int causal,
                  const uint8_t* block_mask) {
  for (int i = 0; i < nin; ++i)
    if (!in[i]) return FA_ERR_NULL;
  for (int i = 0; i < nout; ++i)
    if (!out[i]) return FA_ERR_NULL;
  long long elems = 0;
  int st = check_common(B, H, N, d, scale, causal, block_mask, true, &elems);
  if (st != FA_OK) return st;
  for (int i = 0; i < nin; ++i)
    if (!aligned16(in[i])) return FA_ERR_ALIGN;
  for (int i = 0; i < nout; ++i)
    if (!aligned16(out[i])) return FA_ERR_ALIGN;
  Range ri[9], ro[3];
  for (int i = 0; i < nin; ++i) ri[i] = rng(in[i], in_bytes[i]);
  const long long nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  ri[nin] = rng(block_mask, block_mask ? nb * nb : 0);
  for (int i = 0; i < nout; ++i) ro[i] = rng(out[i], out_bytes[i]);
  return check_alias(ri, nin + 1, ro, nout);
}

fa::FwdArgs fwd_args(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                     float scale, int causal, const uint8_t* block_mask) {
  fa::FwdArgs a = {};
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.mask = block_mask;
  a.N = N;
  a.d = d;
  a.BH = B * H;
  a.nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = std::fabs(scale) * fa::kLog2e;
  a.qsign = scale < 0.f ? 0x80008000u : 0u;
  a.splits = 1;
  return a;
}

size_t splitkv_workspace_bytes(int B, int H, int N, int d, int splits) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128) || splits < 1 || splits > FA_MAX_SPLITS) return 0;
  return fa::splitkv_ws_bytes((long long)B * H, N, d, splits);
}

fa::BwdArgs stage_args(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, const void* workspace, void* dq, void* dk, void* dv, int B, int H, int N,
                       int d, float scale, int causal, const uint8_t* block_mask) {
  fa::BwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<const __bf16*>(o);
  a.dout = static_cast<const __bf16*>(dout);
  a.lse = lse;
  a.dq = static_cast<__bf16*>(dq);
  a.dk = static_cast<__bf16*>(dk);
  a.dv = static_cast<__bf16*>(dv);
  a.delta = static_cast<float*>(const_cast<void*>(workspace));
  a.mask = block_mask;
  a.N = N;
  a.d = d;
  a.BH = B * H;
  a.nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = std::fabs(scale) * fa::kLog2e;
  a.ssign = scale < 0.f ? 0x80008000u : 0u;
  return a;
}

}  // namespace

extern "C" {

const char* flash_attn_status_string(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape (B, H, N must be >= 1; sizes must fit; mask blocks <= limit)";
    case FA_ERR_HEADDIM: return "head dimension d must be 64 or 128";
    case FA_ERR_ALIGN: return "a tensor or workspace pointer is not 16-byte aligned";
    case FA_ERR_SCALE: return "scale must be finite and nonzero";
    case FA_ERR_WORKSPACE: return "workspace is NULL or smaller than flash_attn_bwd_workspace_bytes()";
    case FA_ERR_HIP: return "a HIP kernel launch failed";
    case FA_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA_ERR_FLAG: return "causal must be 0 or 1";
    case FA_ERR_SPLITS: return "splits / parts must be in 1 .. FA_MAX_SPLITS";
    case FA_ERR_UNSUPPORTED: return "option not supported by this entry point (see its declaration)";
    case FA_ERR_SCRATCH: return "B * H * N exceeds FA_NOALLOC_MAX_ROWS, the fixed scratch of flash_attn_bwd_noalloc";
    default: return "unknown status";
  }
}

size_t flash_attn_bwd_workspace_bytes(int B, int H, int N, int d) { return workspace_bytes(B, H, N, d); }

int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, const uint8_t* block_mask, hipStream_t stream) {
  long long elems = 0;
  const __bf16* qb = static_cast<const __bf16*>(q);
  const __bf16* kb = static_cast<const __bf16*>(k);
  const __bf16* vb = static_cast<const __bf16*>(v);
  __bf16* ob = static_cast<__bf16*>(o);
  int st = fwd_checked(qb, kb, vb, ob, lse, B, H, N, d, scale, causal, block_mask, true, &elems);
  if (st != FA_OK) return st;
  return status_of(fa::launch_fwd_bf16(fwd_args(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask), stream));
}

int flash_attn_fwd_pingpong(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                            int d, float scale, int causal, const uint8_t* block_mask, hipStream_t stream) {
  long long elems = 0;
  int st = fwd_checked(static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                       static_cast<__bf16*>(o), lse, B, H, N, d, scale, causal, block_mask, true, &elems);
  if (st != FA_OK) return st;
  if (d != 128 || block_mask) return FA_ERR_UNSUPPORTED;
  return status_of(
      fa::launch_fwd_pingpong_bf16(fwd_args(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask), stream));
}

size_t flash_attn_fwd_splitkv_workspace_bytes(int B, int H, int N, int d, int splits) {
  return splitkv_workspace_bytes(B, H, N, d, splits);
}

int flash_attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                           int d, float scale, int causal, const uint8_t* block_mask, int splits, void* workspace,
                           size_t workspace_bytes_, hipStream_t stream) {
  long long elems = 0;
  int st = fwd_checked(static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                       static_cast<__bf16*>(o), lse, B, H, N, d, scale, causal, block_mask, true, &elems);
  if (st != FA_OK) return st;
  if (splits < 1 || splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  const size_t need = splitkv_workspace_bytes(B, H, N, d, splits);
  if (!workspace || workspace_bytes_ < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  const long long tb = elems * 2, lb = (long long)B * H * N * 4;
  const long long nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  Range in[4] = {rng(q, tb), rng(k, tb), rng(v, tb), rng(block_mask, block_mask ? nb * nb : 0)};
  Range out[3] = {rng(o, tb), rng(lse, lb), rng(workspace, (long long)need)};
  st = check_alias(in, 4, out, 3);
  if (st != FA_OK) return st;
  fa::FwdArgs a = fwd_args(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask);
  a.splits = splits;
  a.o_part = static_cast<float*>(workspace);
  a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        fa::splitkv_o_bytes((long long)B * H, N, d, splits));
  return status_of(fa::launch_fwd_splitkv_bf16(a, stream));
}

int flash_attn_merge(const float* o_parts, const float* lse_parts, int parts, int64_t rows, int d, void* o,
                     float* lse, hipStream_t stream) {
  if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_NULL;
  if (rows < 1 || rows >= kMaxElems / 1024) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (parts < 1 || parts > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  const long long ob = (long long)parts * rows * d * 4, lb = (long long)parts * rows * 4;
  Range in[2] = {rng(o_parts, ob), rng(lse_parts, lb)};
  Range out[2] = {rng(o, rows * d * 2), rng(lse, rows * 4)};
  int st = check_alias(in, 2, out, 2);
  if (st != FA_OK) return st;
  return status_of(fa::launch_merge_bf16(o_parts, lse_parts, parts, rows, d, static_cast<__bf16*>(o), lse, stream));
}

int64_t flash_attn_mxfp8_vt_cols(int N) { return N < 1 ? 0 : (int64_t)fa::fp8_vt_cols(N); }

int flash_attn_fwd_mxfp8(const uint8_t* q8, const uint8_t* q_scales, const uint8_t* k8, const uint8_t* k_scales,
                         const uint8_t* vt8, const uint8_t* vt_scales, void* o, float* lse, int B, int H, int N, int d,
                         float scale, int causal, const uint8_t* block_mask, hipStream_t stream) {
  if (!q8 || !q_scales || !k8 || !k_scales || !vt8 || !vt_scales || !o || !lse) return FA_ERR_NULL;
  long long elems = 0;
  int st = check_common(B, H, N, d, scale, causal, block_mask, true, &elems);
  if (st != FA_OK) return st;
  const void* ptrs[] = {q8, q_scales, k8, k_scales, vt8, vt_scales, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  const long long bh = (long long)B * H, np = fa::fp8_vt_cols(N);
  const long long cb = elems, sb = elems / 32, vtb = bh * d * np, vsb = bh * np * (d / 32);
  const long long nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  Range in[7] = {rng(q8, cb),  rng(q_scales, sb),  rng(k8, cb), rng(k_scales, sb),
                 rng(vt8, vtb), rng(vt_scales, vsb), rng(block_mask, block_mask ? nb * nb : 0)};
  Range out[2] = {rng(o, elems * 2), rng(lse, bh * N * 4)};
  st = check_alias(in, 7, out, 2);
  if (st != FA_OK) return st;
  fa::Fp8FwdArgs a = {};
  a.q8 = q8;
  a.qs = q_scales;
  a.k8 = k8;
  a.ks = k_scales;
  a.vt8 = vt8;
  a.vts = vt_scales;
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.mask = block_mask;
  a.N = N;
  a.Np = (int)np;
  a.d = d;
  a.BH = (int)bh;
  a.nb = (int)nb;
  a.causal = causal;
  a.scale_log2 = std::fabs(scale) * fa::kLog2e;
  a.qsign = scale < 0.f ? 0x80808080u : 0u;
  return status_of(fa::launch_fwd_mxfp8(a, stream));
}

int flash_attn_mxfp8_quantize_rows(const void* x, uint8_t* codes, uint8_t* scales, int B, int H, int N, int d,
                                   hipStream_t stream) {
  if (!x || !codes || !scales) return FA_ERR_NULL;
  long long elems = 0;
  int st = check_common(B, H, N, d, 1.0f, 0, nullptr, true, &elems);
  if (st != FA_OK) return st;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return FA_ERR_ALIGN;
  Range in[1] = {rng(x, elems * 2)};
  Range out[2] = {rng(codes, elems), rng(scales, elems / 32)};
  st = check_alias(in, 1, out, 2);
  if (st != FA_OK) return st;
  return status_of(
      fa::launch_mxfp8_quantize_rows(static_cast<const __bf16*>(x), codes, scales, (long long)B * H * N, d, stream));
}

int flash_attn_mxfp8_quantize_vt(const void* v, uint8_t* codes_t, uint8_t* scales_t, int B, int H, int N, int d,
                                 hipStream_t stream) {
  if (!v || !codes_t || !scales_t) return FA_ERR_NULL;
  long long elems = 0;
  int st = check_common(B, H, N, d, 1.0f, 0, nullptr, true, &elems);
  if (st != FA_OK) return st;
  if ((long long)B * H > 65535) return FA_ERR_SHAPE;  // heads on grid.y
  if (!aligned16(v) || !aligned16(codes_t) || !aligned16(scales_t)) return FA_ERR_ALIGN;
  const long long bh = (long long)B * H, np = fa::fp8_vt_cols(N);
  Range in[1] = {rng(v, elems * 2)};
  Range out[2] = {rng(codes_t, bh * d * np), rng(scales_t, bh * np * (d / 32))};
  st = check_alias(in, 1, out, 2);
  if (st != FA_OK) return st;
  return status_of(fa::launch_mxfp8_quantize_vt(static_cast<const __bf16*>(v), codes_t, scales_t, (int)bh, N, d, stream));
}

int flash_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
                       int d, float scale, int causal, const uint8_t* block_mask, hipStream_t stream) {
  long long elems = 0;
  int st = fwd_checked(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask, false, &elems);
  if (st != FA_OK) return st;
  fa::F32Args a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.out_o = o;
  a.lse = lse;
  a.mask = block_mask;
  a.N = N;
  a.d = d;
  a.BH = B * H;
  a.nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  a.causal = causal;
  a.scale = scale;
  return status_of(fa::launch_fwd_f32(a, stream));
}

int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes_, int B, int H, int N, int d,
                   float scale, int causal, const uint8_t* block_mask, hipStream_t stream) {
  long long elems = 0;
  int st = bwd_checked(static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                       static_cast<const __bf16*>(o), static_cast<const __bf16*>(dout), lse,
                       static_cast<__bf16*>(dq), static_cast<__bf16*>(dk), static_cast<__bf16*>(dv), workspace,
                       workspace_bytes_, B, H, N, d, scale, causal, block_mask, true, &elems);
  if (st != FA_OK) return st;
  const fa::BwdArgs a = stage_args(q, k, v, o, dout, lse, workspace, dq, dk, dv, B, H, N, d, scale, causal, block_mask);
  return status_of(fa::launch_bwd_bf16(a, stream));
}

int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                           int causal, const uint8_t* block_mask, hipStream_t stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  long long elems = 0;
  int st = check_common(B, H, N, d, scale, causal, block_mask, true, &elems);
  if (st != FA_OK) return st;
  if ((long long)B * H * N > fa::kNoallocMaxRows) return FA_ERR_SCRATCH;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  const long long tb = elems * 2, lb = (long long)B * H * N * 4;
  const long long nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  Range in[7] = {rng(q, tb),    rng(k, tb),   rng(v, tb), rng(o, tb), rng(dout, tb), rng(lse, lb),
                 rng(block_mask, block_mask ? nb * nb : 0)};
  Range out[3] = {rng(dq, tb), rng(dk, tb), rng(dv, tb)};
  st = check_alias(in, 7, out, 3);
  if (st != FA_OK) return st;
  void* scratch = nullptr;  // this device's address of the library's fixed array
  if (fa::noalloc_scratch(&scratch) != hipSuccess) return FA_ERR_HIP;
  const fa::BwdArgs a = stage_args(q, k, v, o, dout, lse, scratch, dq, dk, dv, B, H, N, d, scale, causal, block_mask);
  return status_of(fa::launch_bwd_bf16(a, stream));
}

size_t flash_attn_bwd_onepass_workspace_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d != 128) return 0;
  return fa::ws_bytes((long long)B * H, N) + fa::dq_acc_bytes((long long)B * H, N, d);
}

int flash_attn_bwd_onepass(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes_,
                           int B, int H, int N, int d, float scale, int causal, const uint8_t* block_mask,
                           hipStream_t stream) {
  long long elems = 0;
  int st = bwd_checked(static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                       static_cast<const __bf16*>(o), static_cast<const __bf16*>(dout), lse,
                       static_cast<__bf16*>(dq), static_cast<__bf16*>(dk), static_cast<__bf16*>(dv), workspace,
                       workspace_bytes_, B, H, N, d, scale, causal, block_mask, true, &elems);
  if (st != FA_OK) return st;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  const size_t need = flash_attn_bwd_onepass_workspace_bytes(B, H, N, d);
  if (workspace_bytes_ < need) return FA_ERR_WORKSPACE;
  const long long tb = elems * 2, lb = (long long)B * H * N * 4;
  const long long nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  Range in[7] = {rng(q, tb),    rng(k, tb),   rng(v, tb), rng(o, tb), rng(dout, tb), rng(lse, lb),
                 rng(block_mask, block_mask ? nb * nb : 0)};
  Range out[4] = {rng(dq, tb), rng(dk, tb), rng(dv, tb), rng(workspace, (long long)need)};
  st = check_alias(in, 7, out, 4);
  if (st != FA_OK) return st;
  const fa::BwdArgs a = stage_args(q, k, v, o, dout, lse, workspace, dq, dk, dv, B, H, N, d, scale, causal, block_mask);
  float* dq_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + fa::ws_bytes((long long)B * H, N));
  return status_of(fa::launch_bwd_onepass_bf16(a, dq_acc, stream));
}

int flash_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* dout,
                       const float* lse, float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes_,
                       int B, int H, int N, int d, float scale, int causal, const uint8_t* block_mask,
                       hipStream_t stream) {
  long long elems = 0;
  int st = bwd_checked(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes_, B, H, N, d, scale, causal,
                       block_mask, false, &elems);
  if (st != FA_OK) return st;
  fa::F32Args a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = const_cast<float*>(lse);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = static_cast<float*>(workspace);
  a.mask = block_mask;
  a.N = N;
  a.d = d;
  a.BH = B * H;
  a.nb = (N + FA_MASK_BLOCK - 1) / FA_MASK_BLOCK;
  a.causal = causal;
  a.scale = scale;
  return status_of(fa::launch_bwd_f32(a, stream));
}

int flash_attn_bwd_preprocess(const void* q, const void* o, const void* dout, void* workspace,
                              size_t workspace_bytes_, int B, int H, int N, int d, hipStream_t stream) {
  const long long tb = (long long)B * H * N * d * 2;
  const void* in[3] = {q, o, dout};
  const long long ib[3] = {tb, tb, tb};
  void* out[1] = {workspace};
  const long long ob[1] = {(long long)workspace_bytes(B, H, N, d)};
  int st = stage_checked(in, ib, 3, out, ob, 1, B, H, N, d, 1.0f, 0, nullptr);
  if (st != FA_OK) return st;
  if (workspace_bytes_ < workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
  const fa::BwdArgs a = stage_args(q, nullptr, nullptr, o, dout, nullptr, workspace, nullptr, nullptr, nullptr, B, H,
                                   N, d, 1.0f, 0, nullptr);
  return status_of(fa::launch_bwd_delta_bf16(a, stream));
}

int flash_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                        const void* workspace, size_t workspace_bytes_, void* dk, void* dv, int B, int H, int N,
                        int d, float scale, int causal, const uint8_t* block_mask, hipStream_t stream) {
  const long long tb = (long long)B * H * N * d * 2, rb = (long long)B * H * N * 4;
  const void* in[6] = {q, k, v, dout, lse, workspace};
  const long long ib[6] = {tb, tb, tb, tb, rb, (long long)workspace_bytes(B, H, N, d)};
  void* out[2] = {dk, dv};
  const long long ob[2] = {tb, tb};
  int st = stage_checked(in, ib, 6, out, ob, 2, B, H, N, d, scale, causal, block_mask);
  if (st != FA_OK) return st;
  if (workspace_bytes_ < workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
  const fa::BwdArgs a =
      stage_args(q, k, v, nullptr, dout, lse, workspace, nullptr, dk, dv, B, H, N, d, scale, causal, block_mask);
  return status_of(fa::launch_bwd_dkdv_bf16(a, stream));
}

int flash_attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                      const void* workspace, size_t workspace_bytes_, void* dq, int B, int H, int N, int d,
                      float scale, int causal, const uint8_t* block_mask, hipStream_t stream) {
  const long long tb = (long long)B * H * N * d * 2, rb = (long long)B * H * N * 4;
  const void* in[6] = {q, k, v, dout, lse, workspace};
  const long long ib[6] = {tb, tb, tb, tb, rb, (long long)workspace_bytes(B, H, N, d)};
  void* out[1] = {dq};
  const long long ob[1] = {tb};
  int st = stage_checked(in, ib, 6, out, ob, 1, B, H, N, d, scale, causal, block_mask);
  if (st != FA_OK) return st;
  if (workspace_bytes_ < workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
  const fa::BwdArgs a =
      stage_args(q, k, v, nullptr, dout, lse, workspace, dq, nullptr, nullptr, B, H, N, d, scale, causal, block_mask);
  return status_of(fa::launch_bwd_dq_bf16(a, stream));
}

}  // extern "C"
