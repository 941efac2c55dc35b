/*
 * flash_attn.h -- C ABI of the MI355X (gfx950) exact attention forward pass.
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

/* Return codes. Every check runs on the host before anything is launched. */
typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,    /* a required pointer is NULL (with non-empty work)        */
  FA_ERR_SHAPE = -2,   /* B, H or N negative, or a size overflows the kernel's indexing */
  FA_ERR_HEADDIM = -3, /* d is not 64 or 128                                      */
  FA_ERR_DTYPE = -4,   /* dtype is neither FA_BF16 nor FA_FP16                    */
  FA_ERR_SCALE = -5,   /* scale is not finite or not > 0                          */
  FA_ERR_ALIGN = -6,   /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
  FA_ERR_ALIAS = -7,   /* o or lse overlaps an input, or o overlaps lse          */
  FA_ERR_HIP = -8,     /* the HIP runtime reported an error at launch             */
  FA_ERR_ARG = -9      /* causal is not 0 or 1                                    */
} fa_status;

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
 * d       : head dimension, 64 or 128.
 * causal  : 0 for full attention, 1 for causal (top-left aligned: query i sees
 *           keys 0..i).
 * scale   : multiplier of q.k, finite and > 0 (usually 1/sqrt(d)).
 * stream  : hipStream_t (passed as void*) on which the kernel is enqueued; NULL
 *           means the default stream. The call is asynchronous: it returns after
 *           the launch and never synchronises.
 * dtype   : FA_BF16 or FA_FP16.
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

/* Static, never-freed description of a status code (unknown codes included). */
const char* flash_attn_strerror(int status);

/* ABI version of this header, currently 1. */
int flash_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_MI355X_H */
