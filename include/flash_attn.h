/*
 * flash_attn.h — C ABI of an exact tiled scaled-dot-product attention library for AMD MI355X
 * (gfx950).  Forward: S = scale * Q K^T, row softmax and P V fused tile by tile with an online
 * softmax, the N x N score matrix never written to device memory, one log-sum-exp per row
 * returned.  Backward: S and P recomputed tile by tile from that log-sum-exp.
 *
 * Sources (web pages on the method):
 *   [P2] "FlashAttention: how a memory trick unlocked today's giant AI models" (khetwal.com)
 *   [P3] "How FlashAttention Eliminates Transformer Memory Bottlenecks" (Galileo blog)
 *
 * Conventions shared by every entry point
 *   Layout      Q, K, V, O, dO, dQ, dK, dV are contiguous row-major [B, H, N, d] tensors (one
 *               N x d matrix per batch b and head h, as in [P2 "A Worked Example in Pseudocode"]).
 *               LSE is a contiguous [B, H, N] float32 tensor.  All are device pointers, 16-byte
 *               aligned.  Offsets are computed in 64 bits.
 *   Scale       S = scale * Q K^T; scale must be finite and nonzero, of either sign (usually
 *               1/sqrt(d)).  A negative scale is applied exactly: the bf16 and FP8 kernels flip
 *               the sign of the operand they hold in registers (exact) and use |scale| in the
 *               exponent; the fp32 kernels scale each score before taking the row maximum.
 *   Causal      causal = 1 lets query i see key j only when j <= i (square, top-left aligned);
 *               causal = 0 lets every query see every key.
 *   Block mask  block_mask == NULL means dense.  Otherwise a device uint8 array [nb][nb],
 *               nb = ceil(N / 128), row-major, shared by every (b, h): query block I may see key
 *               block J iff block_mask[I * nb + J] != 0.  Masked 128 x 128 tiles are skipped,
 *               never computed ([P3 "Innovation #5: Extension to block-sparse attention
 *               patterns"]).  It combines with causal by AND.  The bf16 entry points accept
 *               nb <= FA_MAX_MASK_BLOCKS.
 *   Dead rows   a query that sees no key gets O = 0, LSE = -inf and contributes no gradient.
 *   Ownership   the caller owns every buffer (including the backward workspace).  The library
 *               allocates no device memory, keeps no state between calls and may be called from
 *               several host threads.  Inputs are read-only and may alias one another; outputs
 *               must not overlap any input or each other (checked: FA_ERR_ALIAS).
 *   Asynchrony  work is enqueued on `stream` (NULL = the default stream) and the call returns
 *               without waiting; results are visible after the stream is synchronised.
 *   Errors      arguments are checked on the host first; on any FA_ERR_* other than FA_ERR_HIP
 *               nothing is enqueued and no output is touched.  FA_ERR_HIP reports a failed
 *               launch (hipGetLastError); some kernels may already be enqueued.  NaN/Inf inside
 *               the inputs are not checked; they propagate to the affected rows.
 */
#ifndef FLASH_ATTN_H
#define FLASH_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_MASK_BLOCK 128
#define FA_MAX_MASK_BLOCKS 2048
#define FA_MAX_SPLITS 64

enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,     /* B, H or N < 1, a size overflows, or nb > FA_MAX_MASK_BLOCKS */
  FA_ERR_HEADDIM = 3,   /* d not in {64, 128} */
  FA_ERR_ALIGN = 4,     /* a tensor or workspace pointer is not 16-byte aligned */
  FA_ERR_SCALE = 5,     /* scale not finite, or zero */
  FA_ERR_WORKSPACE = 6, /* workspace NULL or smaller than flash_attn_bwd_workspace_bytes() */
  FA_ERR_HIP = 7,       /* a kernel launch failed */
  FA_ERR_ALIAS = 8,     /* an output overlaps an input or another output */
  FA_ERR_FLAG = 9,      /* causal not 0 or 1 */
  FA_ERR_SPLITS = 10,   /* splits / parts not in 1 .. FA_MAX_SPLITS */
  FA_ERR_SCRATCH = 11,  /* B * H * N above FA_NOALLOC_MAX_ROWS (flash_attn_bwd_noalloc) */
  FA_ERR_UNSUPPORTED = 12 /* an option the entry point does not support (flash_attn_fwd_pingpong) */
};

/* Forward, bf16 inputs and outputs, fp32 accumulation.
 * Computes, per (b, h), O = softmax(scale * Q K^T restricted to visible keys) V and
 * LSE_i = ln sum_j exp(scale * q_i . k_j) over the visible keys j (natural log).
 * Definition: [P2 "The Quadratic Memory Bottleneck"] (S, P, O); tiling and online softmax:
 * [P2 "Tiling: Breaking the Problem into Pieces", "The Trick: Online Softmax"]; the row
 * statistic kept for the backward pass: [P3 "Innovation #3: Strategic recomputation in the
 * backward pass"].
 *   q, k, v  in   bf16 [B, H, N, d]
 *   o        out  bf16 [B, H, N, d] (round to nearest even)
 *   lse      out  float32 [B, H, N]
 */
int flash_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t *block_mask, hipStream_t stream);

/* Forward, bf16, with the wave-specialised ("ping-pong") schedule instead of the in-wave
 * interleave of flash_attn_fwd: the two waves that share each SIMD alternate between a phase of
 * matrix products (S = K Q^T of one key tile, O += P V of the previous one) and a phase of softmax
 * work (masks, running maximum, rescale, exponentials, row sums), one barrier per phase, so one
 * wave's MFMAs run beside the other's VALU work.  This is the interleaving of matrix products and
 * softmax that "How FlashAttention Bypasses the GPU Memory Bottleneck to Enable Long-Context AI"
 * credits for FlashAttention-3's throughput, done across the two waves of a SIMD.  Same
 * definition, arguments and results as flash_attn_fwd (the same products and sums in the same
 * order: bitwise equal outputs); only d = 128 without a block mask (else FA_ERR_UNSUPPORTED).
 * On MI355X it measures slower than flash_attn_fwd (the operand reads of a whole tile then fall
 * into one phase of each SIMD pair); it is kept as the measured alternative schedule. */
int flash_attn_fwd_pingpong(const void *q, const void *k, const void *v, void *o, float *lse,
                            int B, int H, int N, int d, float scale, int causal,
                            const uint8_t *block_mask, hipStream_t stream);

/* Forward with float32 inputs, outputs and arithmetic (no reduced-precision products).
 * Same definition and arguments as flash_attn_fwd with float tensors. */
int flash_attn_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                       int B, int H, int N, int d, float scale, int causal,
                       const uint8_t *block_mask, hipStream_t stream);

/* Split-key forward, bf16 (the sequence-parallel form of the forward: "How FlashAttention
 * Bypasses the GPU Memory Bottleneck to Enable Long-Context AI" on parallelising over the
 * sequence length).  The 128-key blocks of every (b, h) are cut into `splits` contiguous ranges
 * (range s = blocks [s * nb / splits, (s + 1) * nb / splits), nb = ceil(N / 128)); each range
 * computes its own normalised partial output O_s and log-sum-exp LSE_s over its keys, and the
 * partials are merged exactly as flash_attn_merge does.  The result is flash_attn_fwd's up to
 * floating-point rounding order (not bit-identical).  Worth it when B * H * ceil(N / 128) is
 * small against the GPU's 256 compute units, or when one query block's key range is long.
 *   q, k, v, o, lse, scale, causal, block_mask   as flash_attn_fwd
 *   splits      1 .. FA_MAX_SPLITS (else FA_ERR_SPLITS)
 *   workspace   at least flash_attn_fwd_splitkv_workspace_bytes(B, H, N, d, splits) bytes,
 *               16-byte aligned, owned by the caller; holds the float32 partials
 *               ([splits, B, H, N, d] outputs, then [splits, B, H, N] log-sum-exps); contents
 *               undefined afterwards.  Must not overlap any input or output (FA_ERR_ALIAS).
 */
size_t flash_attn_fwd_splitkv_workspace_bytes(int B, int H, int N, int d, int splits);
int flash_attn_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int N, int d, float scale, int causal,
                           const uint8_t *block_mask, int splits,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/* MX-FP8 forward (the FP8 variant of the forward named in "How FlashAttention Bypasses the GPU
 * Memory Bottleneck to Enable Long-Context AI", on FlashAttention-3).  Same definition as
 * flash_attn_fwd, computed from MX-FP8 inputs (OCP Microscaling Formats v1.0: E4M3 element codes,
 * one E8M0 scale byte 2^(s - 127) per block of 32 consecutive elements along the contraction
 * index) on the scaled FP8 matrix cores, fp32 accumulation and softmax.  The exact result is
 * attention over the dequantised inputs; the kernel adds the rounding of P (values <= 2^8) to
 * E4M3 before the P V product, so each O element is within
 *   sum_j max(2^-4 p_j, 2^-10) |v_j| / sum_j p_j   (p the softmax weights, max_j p_j = 1)
 * of it, plus fp32 rounding; LSE uses P in fp32 and keeps fp32 accuracy.
 *   q8, k8     in  E4M3 codes [B, H, N, d]              (flash_attn_mxfp8_quantize_rows)
 *   q_scales, k_scales  in  E8M0 [B, H, N, d / 32], block c of a row = elements 32c .. 32c + 31
 *   vt8        in  E4M3 codes of V transposed, [B, H, d, Np], Np = flash_attn_mxfp8_vt_cols(N),
 *                  columns >= N zero                    (flash_attn_mxfp8_quantize_vt)
 *   vt_scales  in  E8M0, blocks of 32 keys: scale of feature f, keys 32j .. 32j + 31 of head
 *                  (b, h) at byte (((b H + h) Np/32 + j) 32 + f % 32) (d/32) + f / 32
 *   o          out bf16 [B, H, N, d];  lse  out float32 [B, H, N]
 *   B, H, N, d, scale, causal, block_mask   as flash_attn_fwd
 * All pointers 16-byte aligned device memory; outputs must not overlap inputs (FA_ERR_ALIAS).
 */
int flash_attn_fwd_mxfp8(const uint8_t *q8, const uint8_t *q_scales, const uint8_t *k8,
                         const uint8_t *k_scales, const uint8_t *vt8, const uint8_t *vt_scales,
                         void *o, float *lse, int B, int H, int N, int d, float scale, int causal,
                         const uint8_t *block_mask, hipStream_t stream);

/* MX-FP8 quantisation (OCP MX v1.0, section 6.3) of a bf16 [B, H, N, d] tensor in blocks of 32
 * along d, for Q and K: per block, shared exponent e = floor(log2(max |x|)) - 8 held to
 * [-127, 127] (a zero block takes -127), scale byte e + 127, codes = x * 2^-e rounded to
 * nearest-even E4M3 after clamping to +-448.  Inputs must be finite.
 *   x       in   bf16 [B, H, N, d];  d in {64, 128}
 *   codes   out  E4M3 [B, H, N, d];  scales  out  E8M0 [B, H, N, d / 32]
 */
int flash_attn_mxfp8_quantize_rows(const void *x, uint8_t *codes, uint8_t *scales,
                                   int B, int H, int N, int d, hipStream_t stream);

/* Columns of the transposed V layout: N rounded up to a multiple of 64 (0 if N < 1). */
int64_t flash_attn_mxfp8_vt_cols(int N);

/* MX-FP8 quantisation of V into the transposed layout flash_attn_fwd_mxfp8 reads: blocks of 32
 * consecutive keys per feature, same rule as flash_attn_mxfp8_quantize_rows; keys N .. Np - 1
 * are zero (code 0) and take part in their block as zeros.
 *   v          in   bf16 [B, H, N, d]
 *   codes_t    out  E4M3 [B, H, d, Np];  scales_t  out  E8M0, B * H * Np * d / 32 bytes, laid
 *                   out as described at flash_attn_fwd_mxfp8
 */
int flash_attn_mxfp8_quantize_vt(const void *v, uint8_t *codes_t, uint8_t *scales_t,
                                 int B, int H, int N, int d, hipStream_t stream);

/* Log-sum-exp merge of `parts` partial results computed over disjoint key sets of the same
 * query rows (the partials of a split-key forward, or of key shards held by different
 * devices).  Per row: LSE = ln sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s, the softmax
 * over the union of the key sets; a part with LSE_s = -inf (no visible key) contributes nothing,
 * and a row whose parts are all -inf gets O = 0, LSE = -inf.
 *   o_parts    in   float32 [parts, rows, d], each O_s normalised by its own sum
 *   lse_parts  in   float32 [parts, rows], natural log
 *   parts      1 .. FA_MAX_SPLITS;  rows >= 1;  d in {64, 128}
 *   o          out  bf16 [rows, d] (round to nearest even)
 *   lse        out  float32 [rows]
 */
int flash_attn_merge(const float *o_parts, const float *lse_parts, int parts, int64_t rows, int d,
                     void *o, float *lse, hipStream_t stream);

/* Bytes of device workspace flash_attn_bwd / flash_attn_bwd_f32 need for this shape, or 0 if
 * B, H or N < 1 or d is not 64 or 128.  It holds, per (b, h), D = rowsum(dO * O) as float32 [N]
 * (the size is rounded up to 256 bytes). */
size_t flash_attn_bwd_workspace_bytes(int B, int H, int N, int d);

/* Backward, bf16.  Gradients of L = sum(O * dO) with respect to q, k, v, recomputing S and P
 * tile by tile from lse ([P3 "Innovation #3: Strategic recomputation in the backward pass"]):
 *   D = rowsum(dO * O);  P = exp(scale * Q K^T - LSE);  dV = P^T dO;  dP = dO V^T;
 *   dS = P * (dP - D);   dQ = scale dS K;   dK = scale dS^T Q.
 *   q, k, v     in   bf16 [B, H, N, d]  (the forward's inputs)
 *   o, lse      in   the forward's outputs for the same inputs, scale, causal and block_mask
 *   dout        in   bf16 [B, H, N, d]  (dO)
 *   dq, dk, dv  out  bf16 [B, H, N, d]
 *   workspace   scratch of at least flash_attn_bwd_workspace_bytes(B, H, N, d) bytes, 16-byte
 *               aligned; its contents are undefined afterwards.
 */
int flash_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                   const void *dout, const float *lse,
                   void *dq, void *dk, void *dv,
                   void *workspace, size_t workspace_bytes,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t *block_mask, hipStream_t stream);

/* Backward, bf16, d = 128, in one pass over each key block ([P3 "Innovation #3"]): one
 * recomputation of S and P per (key block, query tile) yields dV, dK and the block's share of dQ,
 * which is added with float32 atomics into an accumulator in the workspace (zeroed by the
 * pre-pass kernel, converted to bf16 times scale at the end).  Same definition, arguments and
 * checks as flash_attn_bwd; dV equals flash_attn_bwd's bit for bit, dK and dQ agree with it up to
 * rounding (dS formed from P in float32; dQ's float32 sums in an order that varies run to run).
 *   workspace   at least flash_attn_bwd_onepass_workspace_bytes(B, H, N, d) bytes, 16-byte
 *               aligned: D (float32 [B, H, N], rounded up to 256 bytes), then the dQ accumulator
 *               (float32 [B, H, N, d]); contents undefined afterwards.
 *   d != 128 gives FA_ERR_UNSUPPORTED. */
size_t flash_attn_bwd_onepass_workspace_bytes(int B, int H, int N, int d);
int flash_attn_bwd_onepass(const void *q, const void *k, const void *v, const void *o,
                           const void *dout, const float *lse,
                           void *dq, void *dk, void *dv,
                           void *workspace, size_t workspace_bytes,
                           int B, int H, int N, int d, float scale, int causal,
                           const uint8_t *block_mask, hipStream_t stream);

/* Backward with float32 tensors and arithmetic; same definition and arguments. */
int flash_attn_bwd_f32(const float *q, const float *k, const float *v, const float *o,
                       const float *dout, const float *lse,
                       float *dq, float *dk, float *dv,
                       void *workspace, size_t workspace_bytes,
                       int B, int H, int N, int d, float scale, int causal,
                       const uint8_t *block_mask, hipStream_t stream);

/* The three stages flash_attn_bwd runs, exposed one by one (bf16) for callers that schedule
 * them themselves or time them separately.  Enqueued in this order on one stream, with one
 * workspace of at least flash_attn_bwd_workspace_bytes() bytes, they produce exactly what
 * flash_attn_bwd produces.  Same conventions and checks as flash_attn_bwd.
 *
 * Stage 1: the pre-pass over rows: D_i = sum_c dO_ic * O_ic (equals rowsum(P * dP)), written
 * into the workspace as float32 [B, H, N].
 *   q, o, dout in bf16 [B, H, N, d]; q is checked like the others but not read. */
int flash_attn_bwd_preprocess(const void *q, const void *o, const void *dout,
                              void *workspace, size_t workspace_bytes,
                              int B, int H, int N, int d, hipStream_t stream);

/* Stage 2: dK and dV, one pass over the query tiles that see each key block (recomputing S and
 * P from lse, [P3 "Innovation #3"]).  Reads the workspace stage 1 wrote.
 *   q, k, v, dout bf16 in; lse float32 in; dk, dv bf16 out. */
int flash_attn_bwd_dkdv(const void *q, const void *k, const void *v, const void *dout,
                        const float *lse, const void *workspace, size_t workspace_bytes,
                        void *dk, void *dv,
                        int B, int H, int N, int d, float scale, int causal,
                        const uint8_t *block_mask, hipStream_t stream);

/* Stage 3: dQ, one pass over the key tiles each query block sees (recomputing S, P and dP).
 * Reads the workspace stage 1 wrote.
 *   q, k, v, dout bf16 in; lse float32 in; dq bf16 out. */
int flash_attn_bwd_dq(const void *q, const void *k, const void *v, const void *dout,
                      const float *lse, const void *workspace, size_t workspace_bytes,
                      void *dq,
                      int B, int H, int N, int d, float scale, int causal,
                      const uint8_t *block_mask, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP stream capture, tight serving
 * loops, harnesses that forbid hipMalloc): flash_attn_bwd without the workspace argument.  The
 * float32 rows of D it needs live in a fixed array inside the library, 16 MiB per device
 * (FA_NOALLOC_MAX_ROWS rows), held from the first call on a device until the process ends; the
 * call allocates and frees nothing.  Same kernels, results, arguments and checks as
 * flash_attn_bwd otherwise.
 *   B * H * N must be <= FA_NOALLOC_MAX_ROWS (else FA_ERR_SCRATCH, nothing enqueued).
 *   Every call on one device shares that device's array: calls whose work overlaps on one device
 *   (on different streams, or from different host threads without ordering) race on it and give
 *   undefined results.  Calls ordered on one stream are safe; every row of D is rewritten by
 *   each call before it is read, so nothing carries over from the previous call.
 *   FA_ERR_HIP also reports a failed lookup of the array's device address.  That lookup
 *   (hipGetSymbolAddress) runs on the first call on each device: make that first call outside
 *   stream capture; later calls make no HIP call but the kernel launches. */
#define FA_NOALLOC_MAX_ROWS 4194304
int flash_attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                           const void *dout, const float *lse,
                           void *dq, void *dk, void *dv,
                           int B, int H, int N, int d, float scale, int causal,
                           const uint8_t *block_mask, hipStream_t stream);

/* Static English text for a status code ("unknown status" for anything else). */
const char *flash_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_H */
