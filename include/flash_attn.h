/*
 * flash_attn.h -- C ABI of the MI355X (gfx950) exact attention forward and
 * backward passes.
 *
 * The operation: for every batch b, head h and query row i,
 *
 *     s_ij   = scale * sum_k q[b,h,i,k] * k[b,h,j,k]
 *     o[b,h,i,:] = sum_j softmax_j(s_i.) * v[b,h,j,:]
 *     lse[b,h,i] = ln sum_j exp(s_ij)
 *
 * with j ranging over 0..N-1, or over 0..i when causal (query i attends keys
 * j <= i). This is scaled dot-product attention as stated in "6.1 FlashAttention
 * V1 in detail", §1.1 (S = QK^T / sqrt(d), P = softmax(S), O = PV) with the scale
 * passed explicitly; the row statistic L = m + log(l) is the one the forward pass
 * keeps for recomputation in the backward pass ("FlashAttention: IO-Aware Tiling,
 * Online Softmax Mathematics, Memory Hierarchy Dynamics, and Kernel Evolution",
 * section "Backward Pass Recomputation"), stored here in natural-log units as a
 * single fp32 value per row. The N x N scores and probabilities are never written
 * to memory: query tiles stream key/value tiles through on-chip memory with a
 * running row maximum, denominator and unnormalised accumulator ("FlashAttention:
 * optimize data movement before counting FLOPs", section 02, The mechanism).
 */
#ifndef FLASH_ATTN_MI355X_H
#define FLASH_ATTN_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. Accumulation is always fp32. */
typedef enum { FA_BF16 = 0, FA_FP16 = 1 } fa_dtype;

/* Layouts written by flash_attn_quantize_fp8. */
typedef enum { FA_FP8_ROWS = 0, FA_FP8_KEYS_T = 1 } fa_fp8_layout;

/* FP8 formats (OCP 8-bit floating point) of flash_attn_quantize_fp8 and
 * flash_attn_fwd_fp8. */
typedef enum { FA_FP8_E4M3 = 0, FA_FP8_E5M2 = 1 } fa_fp8_format;

/* Forward kernels an unsplit call can run (flash_attn_fwd_kernel). */
typedef enum { FA_FWD_KERNEL_PIPELINED = 1, FA_FWD_KERNEL_PINGPONG = 2 } fa_fwd_kernel;

/* Return codes. Every check runs on the host before anything is launched. */
typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,    /* a required pointer is NULL (with non-empty work)        */
  FA_ERR_SHAPE = -2,   /* B, H or N negative, or a size overflows the kernel's indexing */
  FA_ERR_HEADDIM = -3, /* d is not 64, 128 or 256 (strided: a multiple of 8 up to
                          256; key split and FP8: 64 or 128)                     */
  FA_ERR_DTYPE = -4,   /* dtype is neither FA_BF16 nor FA_FP16                    */
  FA_ERR_SCALE = -5,   /* scale is not finite or not > 0                          */
  FA_ERR_ALIGN = -6,   /* a 16-bit tensor not 16-byte aligned, or an fp32 one not 4-byte aligned */
  FA_ERR_ALIAS = -7,   /* an output overlaps an input or another output          */
  FA_ERR_HIP = -8,     /* the HIP runtime reported an error at launch             */
  FA_ERR_ARG = -9,     /* causal is not 0 or 1, num_splits is negative, or an FP8
                          layout or format is not one of the defined values       */
  FA_ERR_WORKSPACE = -10, /* split workspace NULL, not 16-byte aligned or too small */
  FA_ERR_STRIDE = -11, /* strided call: a stride negative, not a multiple of 8 elements, a row
                          stride below d or >= 2^23, a slice spanning >= 2 GiB, or o / lse
                          overlapping itself                                         */
  FA_ERR_SCRATCH = -12 /* flash_attn_fwd_splitkv_noalloc: the split needs more than
                          FA_SPLITKV_SCRATCH_BYTES of partial results             */
} fa_status;

/* Bytes of the library's own device array that flash_attn_fwd_splitkv_noalloc
 * keeps its partial results in (65 MiB per GPU). Every split that
 * flash_attn_fwd_splitkv_plan picks for d <= 128 on a device of up to 256
 * compute units fits: it makes fewer than 2 * cus work items of at most 256
 * rows, so at most 2 * 256 * 256 * 129 * 4 bytes (64.5 MiB) of partials. */
#define FA_SPLITKV_SCRATCH_BYTES (65u * 1024u * 1024u)

/*
 * flash_attn_fwd -- exact attention forward on one stream.
 *
 * q, k, v : device pointers to contiguous [B, H, N, d] tensors of `dtype`
 *           (row-major, d fastest). Read only.
 * o       : device pointer, contiguous [B, H, N, d] of `dtype`; written with the
 *           attention output rounded to nearest-even from fp32.
 * lse     : device pointer, contiguous [B, H, N] fp32; written with the natural-log
 *           log-sum-exp of each row's scaled scores.
 * B, H, N : batch, heads, sequence length (queries and keys share N). Any of them
 *           zero means there is nothing to do: FA_OK is returned and no pointer is
 *           touched. Requires N * d < 2^31 and B * H * ceil(N / 256) < 2^31.
 * d       : head dimension, 64, 128 or 256. With d = 256 the kernel runs twice, once
 *           per 128-column half of v and o; each run recomputes the scores, so the
 *           matrix work is 1.5 times that of one pass.
 * causal  : 0 for full attention, 1 for causal (top-left aligned: query i sees
 *           keys 0..i).
 * scale   : multiplier of q.k, finite and > 0 (usually 1/sqrt(d)).
 * stream  : hipStream_t (passed as void*) on which the kernel is enqueued; NULL
 *           means the default stream. The call is asynchronous: it returns after
 *           the launch and never synchronises.
 * dtype   : FA_BF16 or FA_FP16.
 *
 * Value range: with FA_BF16 a row's probabilities are taken relative to a kept
 * reference that may lie up to 15 (log2 units) below the row's running maximum, so
 * before normalisation they reach 2^15 and the fp32 accumulator sum_j p_j v_j stays
 * finite only while N * max|v| < 2^113 (about 2.5e30 at N = 4096; bf16 itself reaches
 * 3.4e38). Larger values can overflow to inf/NaN in o; they are not detected. With
 * FA_FP16 the reference is the exact running maximum (p <= 1) and every fp16 value
 * is admissible.
 *
 * Ownership: the caller owns every buffer; the library allocates nothing, frees
 * nothing and keeps no pointer after returning. The library holds no state, so
 * concurrent calls on different streams are safe.
 * Errors: returns FA_OK or one of the negative codes above; nothing is launched
 * when a check fails. After a launch, FA_ERR_HIP reports a launch-time error
 * (hipGetLastError); errors during execution surface at the caller's next
 * synchronisation.
 */
int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                   void* stream, int dtype);

/*
 * flash_attn_fwd_validate -- the argument checks of flash_attn_fwd alone.
 * Same arguments and meaning; returns the status flash_attn_fwd would return
 * before launching (FA_OK when it would launch, or when there is nothing to do).
 * Launches nothing, dereferences nothing and makes no HIP call, so it can be
 * used where no GPU is present.
 */
int flash_attn_fwd_validate(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                            void* stream, int dtype);

/*
 * flash_attn_fwd_strided -- flash_attn_fwd on strided views and any head dimension
 * d that is a multiple of 8 up to 256. The tensors are addressed as in the
 * strided kernel interface of "6.1 FlashAttention V1 in detail", §8.3 (a stride
 * per batch, head and row for each of q, k, v, o; batch and head strides for the
 * row statistics), and a head dimension that is not a power of two is handled as
 * that section handles BLOCK_D > D: the kernel works on the next size it is built
 * for (64, 80, 96, 128 or 256) with the positions past d masked, so they add
 * nothing to the scores and are never stored. Above 128 the 256-wide instance runs
 * once per 128 columns of v and o (twice for d > 128).
 *
 * Element (b, h, i, c) of q is q[b*q_strides[0] + h*q_strides[1] + i*q_strides[2] + c]
 * (in elements of `dtype`; the head dimension is contiguous), likewise k, v and o;
 * lse[b, h, i] is lse[b*lse_strides[0] + h*lse_strides[1] + i] (fp32 elements).
 * q_strides, k_strides, v_strides, o_strides: host arrays of 3 int64 (batch, head,
 * row); lse_strides: host array of 2 int64 (batch, head). Read during the call only.
 * Every other argument and the result are as for flash_attn_fwd.
 *
 * Requirements (FA_ERR_STRIDE otherwise): all strides >= 0; the strides of q, k,
 * v and o multiples of 8 elements (so every row starts 16-byte aligned); each row
 * stride >= d and < 2^23; ((N - 1) * row stride + d) * 2 < 2^31 bytes per slice;
 * o and lse must not overlap themselves (checked with a sufficient condition:
 * in increasing stride order every dimension of size > 1 steps past the span of
 * the dimensions inside it). Inputs may overlap each other and may repeat
 * (stride 0 shares one K/V head among all heads, for example). d must be a
 * multiple of 8 in [8, 256] (FA_ERR_HEADDIM). o and lse must not overlap any
 * input's span (FA_ERR_ALIAS). Requires B * H * ceil(N / 256) < 2^31.
 */
int flash_attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t N, int64_t d,
                           const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                           const int64_t* o_strides, const int64_t* lse_strides,
                           int causal, float scale, void* stream, int dtype);

/*
 * flash_attn_fwd_strided_validate -- the checks of flash_attn_fwd_strided alone
 * (same arguments, same status); launches nothing and makes no HIP call.
 */
int flash_attn_fwd_strided_validate(const void* q, const void* k, const void* v, void* o, float* lse,
                                    int64_t B, int64_t H, int64_t N, int64_t d,
                                    const int64_t* q_strides, const int64_t* k_strides,
                                    const int64_t* v_strides, const int64_t* o_strides,
                                    const int64_t* lse_strides, int causal, float scale,
                                    void* stream, int dtype);

/*
 * flash_attn_quantize_fp8 -- block quantization of a contiguous [B, H, N, d] bf16 /
 * fp16 tensor to FP8 (E4M3 or E5M2) for flash_attn_fwd_fp8 ("FlashAttention:
 * IO-Aware Tiling, Online Softmax Mathematics, Memory Hierarchy Dynamics, and Kernel
 * Evolution", section on FlashAttention-3: FP8 E4M3/E5M2 with block-level
 * quantization and dynamic scaling factors).
 *
 * A block is 64 consecutive rows (keys) of one (batch, head) slice; T = ceil(N/64)
 * blocks per slice. Block t's scale is 2^e with e the smallest integer such that
 * its largest magnitude a satisfies a <= F * 2^e, F the format's largest finite
 * value (e = 0 for an all-zero block; e limited to [-127, 127]); each value is
 * stored as the OCP code of x / 2^e, rounded to nearest even:
 *   FA_FP8_E4M3: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, F = 448;
 *   FA_FP8_E5M2: 1 sign, 5 exponent bits with bias 15, 2 mantissa bits, F = 57344.
 * The value a code c of block t stands for is decode(c) * 2^e.
 *
 * x           : device, contiguous [B, H, N, d] of `dtype` (FA_BF16 / FA_FP16). Read only.
 * x8          : device, written. layout FA_FP8_ROWS: [B, H, N, d] bytes (row-major,
 *               queries and keys). layout FA_FP8_KEYS_T (values): [B, H, T, d, 64]
 *               bytes; row c of block t holds column c of the block's 64 keys,
 *               position p holding key 32*((p%32)/16) + 8*((p%16)/4) + 4*(p/32) + p%4
 *               of the block (the key order the attention kernel's P operand uses);
 *               keys at or past N are 0.
 * scale_codes : device, written, [B, H, T] int32: e + 127 (the E8M0 code of 2^e).
 * d           : 64 or 128.  layout: FA_FP8_ROWS or FA_FP8_KEYS_T (else FA_ERR_ARG).
 * format      : FA_FP8_E4M3 or FA_FP8_E5M2 (else FA_ERR_ARG).
 * stream, ownership, errors: as for flash_attn_fwd. Alignment: x and x8 16 bytes,
 * scale_codes 4 (FA_ERR_ALIGN); x8 and scale_codes must not overlap x or each
 * other (FA_ERR_ALIAS). Requires N * d < 2^31 and B * H * T < 2^31.
 */
int flash_attn_quantize_fp8(const void* x, void* x8, int32_t* scale_codes, int64_t B, int64_t H, int64_t N,
                            int64_t d, int layout, void* stream, int dtype, int format);

/* flash_attn_quantize_fp8_validate -- its checks alone; no HIP call. */
int flash_attn_quantize_fp8_validate(const void* x, void* x8, int32_t* scale_codes, int64_t B, int64_t H,
                                     int64_t N, int64_t d, int layout, void* stream, int dtype, int format);

/*
 * flash_attn_fwd_fp8 -- the attention forward on FP8 inputs: o and lse are the
 * attention of the dequantized q, k, v (o as for flash_attn_fwd, in out_dtype;
 * lse in fp32, natural log). Both products run on the CDNA4 scaled FP8 matrix
 * instruction with the blocks' scales applied exactly; the probabilities P are
 * rounded to E4M3 for the P V product (relative to the row maximum, times 2^8),
 * while the row sums use them unrounded.
 *
 * q8, k8  : device, [B, H, N, d] FP8 codes from flash_attn_quantize_fp8 (FA_FP8_ROWS).
 * v8t     : device, [B, H, T, d, 64] FP8 codes from flash_attn_quantize_fp8 (FA_FP8_KEYS_T).
 * q_scale, k_scale, v_scale : device, [B, H, T] int32 scale codes of q8, k8, v8t.
 * o       : device, written, contiguous [B, H, N, d] of out_dtype.
 * lse     : device, written, contiguous [B, H, N] fp32.
 * d       : 64 or 128 (FA_ERR_HEADDIM otherwise). causal, scale, stream: as for flash_attn_fwd.
 * out_dtype : FA_BF16 or FA_FP16.
 * format  : FA_FP8_E4M3 or FA_FP8_E5M2, the format of q8, k8 and v8t (all three;
 *           else FA_ERR_ARG). P is rounded to E4M3 in either case.
 * Ownership and errors as for flash_attn_fwd; 16-byte alignment for q8, k8, v8t, o
 * and 4 for the scale arrays and lse; o and lse must not overlap an input or each
 * other.
 */
int flash_attn_fwd_fp8(const void* q8, const void* k8, const void* v8t, const int32_t* q_scale,
                       const int32_t* k_scale, const int32_t* v_scale, void* o, float* lse,
                       int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                       void* stream, int out_dtype, int format);

/* flash_attn_fwd_fp8_validate -- its checks alone; no HIP call. */
int flash_attn_fwd_fp8_validate(const void* q8, const void* k8, const void* v8t, const int32_t* q_scale,
                                const int32_t* k_scale, const int32_t* v_scale, void* o, float* lse,
                                int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                                void* stream, int out_dtype, int format);

/*
 * flash_attn_fwd_splitkv -- the forward pass with every query tile's keys cut
 * into num_splits contiguous ranges processed as separate work items, for shapes
 * with fewer (batch, head, 256-row query tile) items than the GPU has compute
 * units. Each range produces, per query row, its own softmax statistics and
 * normalised output; a second kernel merges the ranges of each row with the
 * two-block rule of "FlashAttention: IO-Aware Tiling, Online Softmax
 * Mathematics, Memory Hierarchy Dynamics, and Kernel Evolution", section
 * "Online Softmax Mathematics" (m = max(m1, m2), l = e^(m1-m) l1 + e^(m2-m) l2,
 * O = (l1 e^(m1-m) / l) O1 + (e^(m2-m) / l) P2 V2), applied to all ranges at once.
 * The result is the same attention as flash_attn_fwd (o and lse as documented
 * there), up to rounding.
 *
 * Arguments q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype: as for
 * flash_attn_fwd, except that d is 64 or 128 (FA_ERR_HEADDIM otherwise).
 * num_splits : ranges per query tile. 0 chooses with flash_attn_fwd_splitkv_plan
 *           for the current device; values above the largest useful count (no
 *           empty range: the fewest 64-key tiles any query tile visits, at most
 *           16) are reduced to it. A resolved count of 1 runs flash_attn_fwd and
 *           leaves the workspace untouched (it may then be NULL).
 * workspace : device memory owned by the caller, 16-byte aligned, at least
 *           flash_attn_fwd_splitkv_workspace_size(...) bytes for the resolved
 *           count S. On return it holds fp32 partial outputs [S, B*H, N, d]
 *           followed by fp32 partial log-sum-exps [S, B*H, N] (range s of a row:
 *           its keys' normalised output and ln of its sum of exp(scores); a row
 *           with no visible key in the range has output 0 and -inf). It must not
 *           overlap q, k, v, o or lse (FA_ERR_ALIAS) and must not be shared with
 *           a concurrent call.
 * workspace_bytes : size of workspace in bytes (FA_ERR_WORKSPACE if too small).
 *
 * Ownership, streams and errors as for flash_attn_fwd (two kernels are enqueued
 * on `stream` when S > 1). With num_splits = 0 the call queries the current
 * device's compute-unit count (one HIP attribute query per device, cached).
 * Requires B * H * ceil(N / 256) * S < 2^31.
 */
int flash_attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                           int num_splits, void* workspace, uint64_t workspace_bytes,
                           void* stream, int dtype);

/*
 * flash_attn_fwd_splitkv_validate -- the checks of flash_attn_fwd_splitkv alone;
 * no HIP call. With num_splits = 0 the workspace is not checked (the count is
 * chosen at launch).
 */
int flash_attn_fwd_splitkv_validate(const void* q, const void* k, const void* v, void* o, float* lse,
                                    int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                                    int num_splits, void* workspace, uint64_t workspace_bytes,
                                    void* stream, int dtype);

/*
 * flash_attn_fwd_splitkv_plan -- the split count chosen for a device with `cus`
 * compute units: 1 when B * H * ceil(N / 256) >= cus or N <= 448 (fewer than 8
 * key tiles: the merge launch would cost more than the split saves), else
 * ceil(cus / items) reduced to the largest useful count (see num_splits above).
 * Pure function (no
 * HIP call). Returns the count (>= 1) or a negative status for invalid shapes
 * (FA_ERR_SHAPE, FA_ERR_HEADDIM, FA_ERR_ARG).
 */
int flash_attn_fwd_splitkv_plan(int64_t B, int64_t H, int64_t N, int64_t d, int causal, int cus);

/*
 * flash_attn_fwd_splitkv_workspace_size -- workspace bytes flash_attn_fwd_splitkv
 * needs for num_splits (>= 1; reduced as above): S * B * H * N * (d + 1) * 4 for
 * the resolved S > 1, and 0 when S resolves to 1 or the shape is empty. Negative
 * status for invalid arguments. Pure function.
 */
int64_t flash_attn_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                                              int num_splits);

/*
 * flash_attn_fwd_splitkv_noalloc -- flash_attn_fwd_splitkv for callers that cannot
 * allocate device memory at the call (code under stream capture, serving loops or
 * harnesses that forbid allocation): the same computation, kernels and result,
 * with the partial outputs and log-sum-exps kept in a device array of the library
 * (FA_SPLITKV_SCRATCH_BYTES, one copy per GPU, held from the first use of the
 * library on that GPU until the process ends) instead of a caller workspace.
 *
 * Arguments q, k, v, o, lse, B, H, N, d, causal, scale, num_splits, stream, dtype:
 * as for flash_attn_fwd_splitkv. The call allocates and frees nothing; on the
 * first call on a device it looks up that device's copy of the array (the current
 * device at the call).
 * Errors: as for flash_attn_fwd_splitkv, plus FA_ERR_SCRATCH when the resolved
 * split needs more than FA_SPLITKV_SCRATCH_BYTES (nothing is launched), and
 * FA_ERR_HIP when the array's address cannot be obtained. A resolved count of 1
 * runs flash_attn_fwd and leaves the array untouched.
 * Concurrency: every call on one GPU shares that GPU's array, and a call leaves
 * its partials there; calls that overlap in time on one GPU (different streams,
 * or host threads without ordering between their streams) race and may return
 * wrong results. Calls ordered on one stream are safe: nothing in the array needs
 * clearing between them, since each call writes every partial it reads.
 */
int flash_attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                                   int num_splits, void* stream, int dtype);

/*
 * flash_attn_bwd -- gradients of the forward pass with respect to q, k and v.
 *
 * For the loss gradient dout = dL/do of o = flash_attn_fwd(q, k, v), with
 * S = scale * q k^T (masked like the forward) and P = softmax(S) row by row:
 *
 *     dv = P^T dout,  dP = dout v^T,  dS = P o (dP - D),  dq = scale * dS k,
 *     dk = scale * dS^T q,   D_i = rowsum(dout o o)_i   ("o" elementwise)
 *
 * ("6.1 FlashAttention V1 in detail", §6.1 and §6.2; "FlashAttention: IO-Aware
 * Tiling, Online Softmax Mathematics, Memory Hierarchy Dynamics, and Kernel
 * Evolution", section "Backward Pass Recomputation", where scale = 1/sqrt(d)).
 * P is rebuilt tile by tile from q, k and lse (P = exp(S - lse)); no N x N
 * matrix is ever written to memory.
 *
 * q, k, v : device, contiguous [B, H, N, d] of `dtype`, the forward's inputs. Read only.
 * o       : device, contiguous [B, H, N, d] of `dtype`, the forward's output. Read only.
 * dout    : device, contiguous [B, H, N, d] of `dtype`. Read only.
 * lse     : device, contiguous [B, H, N] fp32, the forward's lse. Read only.
 * dq, dk, dv : device, contiguous [B, H, N, d] of `dtype`; written, rounded to
 *           nearest-even from fp32.
 * delta   : device, contiguous [B, H, N] fp32 workspace owned by the caller;
 *           written with D (the kernels read it back), so it must not be shared
 *           with a concurrent call.
 * B, H, N, d, causal, scale, stream, dtype: as for flash_attn_fwd, and they must
 *           be the values the forward ran with. Requires N * d < 2^31 and
 *           B * H * ceil(N / 128) < 2^31.
 *
 * Ownership, streams and errors as for flash_attn_fwd: nothing is allocated,
 * two kernels are enqueued on `stream` and nothing is synchronised. Alignment:
 * the 16-bit tensors 16-byte aligned, lse and delta 4-byte aligned
 * (FA_ERR_ALIGN). dq, dk, dv and delta must not overlap each other or any input
 * (FA_ERR_ALIAS).
 */
int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, float* delta,
                   int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                   void* stream, int dtype);

/*
 * flash_attn_bwd_validate -- the argument checks of flash_attn_bwd alone (same
 * arguments, same status); launches nothing and makes no HIP call.
 */
int flash_attn_bwd_validate(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, float* delta,
                            int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                            void* stream, int dtype);

/*
 * flash_attn_fwd_kernel -- which forward kernel flash_attn_fwd, flash_attn_fwd_strided
 * and an unsplit flash_attn_fwd_splitkv call launch for sequence length N, head
 * dimension d and mask `causal`. Both compute the same tiled online-softmax forward
 * ("FlashAttention: optimize data movement before counting FLOPs", section 02, The
 * mechanism) over 256-row query tiles; they differ in how the scores' softmax is
 * overlapped with the matrix products. FA_FWD_KERNEL_PIPELINED software-pipelines
 * each wave (scores of key tile t + 1 and the product of tile t - 1 around the
 * softmax of tile t); FA_FWD_KERNEL_PINGPONG lets the two waves of a SIMD alternate.
 * The ping-pong kernel serves d <= 64, d in 97..128 and d in 129..256 (its 64-,
 * 128- and 256-wide instances); the pipelined kernel serves d in 65..96 (80- and
 * 96-wide instances).
 * The choice does not depend on N or the mask today; both arguments are checked
 * and kept so that it may. The environment variable FLASH_ATTN_FWD_KERNEL, read at
 * every call, forces one: "pipelined" or "pingpong" (then d in 65..96 runs the
 * ping-pong kernel's 128-wide instance); d above 128 always takes the ping-pong kernel.
 * N     : sequence length, >= 0 (else FA_ERR_SHAPE).
 * d     : head dimension, a multiple of 8 in 8..256 (else FA_ERR_HEADDIM).
 * causal: 0 or 1 (else FA_ERR_ARG).
 * Returns FA_FWD_KERNEL_PIPELINED or FA_FWD_KERNEL_PINGPONG, or the negative status.
 * Makes no HIP call and keeps no state.
 */
int flash_attn_fwd_kernel(int64_t N, int64_t d, int causal);

/* Static, never-freed description of a status code (unknown codes included). */
const char* flash_attn_strerror(int status);

/* ABI version of this header, currently 9 (1: forward only; 2: + backward;
 * 3: + key-split forward; 4: + strided forward; 5: + FP8 quantization and forward;
 * 6: + key-split forward without a caller workspace; 7: FP8 format argument, E5M2;
 * 8: + forward kernel query; 9: head dimensions up to 256 in the forward). */
int flash_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_MI355X_H */
