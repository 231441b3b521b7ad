/*
 * attn_fwd.h -- C ABI of the MI355X (gfx950) fused scaled-dot-product attention forward.
 *
 * What is computed (per batch b and head h, on row-major [batch, heads, L, D] tensors):
 *
 *   S[i, j] = sm_scale * sum_d Q[i, d] * K[j, d]
 *   O[i, :] = sum_{j visible from i} exp(S[i, j] - m_i) * V[j, :]  /  sum_{j visible} exp(S[i, j] - m_i)
 *
 * with m_i the largest visible score of row i.  The kernels reach this with the
 * FlashAttention-2 online softmax: a running row maximum, a running exp-sum and a
 * rescaled fp32 accumulator, finished by O = acc / l ("Triton-CUDA Attention",
 * online-softmax core and full example; "Fused Attention", _attn_fwd_inner and
 * _attn_fwd).  Exponentials are taken base 2 with log2(e) folded into the scale
 * ("Triton-CUDA Attention", online-softmax core).
 *
 * Mask modes:
 *   ATTN_MASK_NONE        every key is visible ("Triton-CUDA Attention", full example).
 *   ATTN_MASK_CAUSAL      key j is visible from query i when j <= i; key tiles left of the
 *                         query block run unmasked, the diagonal tiles masked ("Fused
 *                         Attention", _attn_fwd_inner stages 1 and 2).
 *   ATTN_MASK_BLOCK_DIAG  only the block_size x block_size diagonal blocks of the score
 *                         matrix exist; each block is one tile with an exact (not online)
 *                         softmax ("TLX Block Attention", problem statement and kernel).
 *
 * Memory: q, k, v, o are device pointers owned by the caller, each a contiguous
 * [batch, heads, L, D] array (D fastest), the layout every page uses, starting on a
 * 16-byte boundary (as every HIP allocation does).  o has Q's element type and must not
 * overlap q, k or v.  The library allocates nothing,
 * frees nothing and never synchronises: the work is enqueued on `stream` (a
 * hipStream_t; NULL is the default stream) and the call returns.
 *
 * Errors: all arguments are validated on the host before any HIP call; on an error
 * nothing is enqueued and o is untouched.  Launch failures reported by the HIP
 * runtime right after the launch return ATTN_ERR_HIP; faults during execution
 * surface at the caller's next synchronisation.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 2

typedef enum {
    ATTN_MASK_NONE = 0,
    ATTN_MASK_CAUSAL = 1,
    ATTN_MASK_BLOCK_DIAG = 2
} attn_mask_t;

typedef enum {
    ATTN_F16 = 0,          /* Q, K, V, O binary16; P rounded to binary16 before P.V          */
    ATTN_BF16 = 1,         /* Q, K, V, O bfloat16; P rounded to bfloat16 before P.V          */
    ATTN_BF16_V_E5M2 = 2,  /* Q, K, O bfloat16; V OCP fp8 e5m2; P rounded to e5m2 before P.V
                              and the row sum taken over the unrounded P ("Fused Attention",
                              _attn_fwd_inner, fp8 branch)                                   */
    ATTN_F16_V_E5M2 = 3    /* the same with Q, K, O binary16 (the fp8 branch keys only on V's
                              type)                                                          */
} attn_dtype_t;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,         /* a required pointer is NULL                                   */
    ATTN_ERR_SHAPE = 2,        /* negative size, size overflow, block_size not dividing L, or a
                                  pointer or stride off its required boundary                   */
    ATTN_ERR_UNSUPPORTED = 3,  /* (mode, D, dtype, block_size) outside the supported set        */
    ATTN_ERR_HIP = 4,          /* the HIP runtime reported an error at launch                   */
    ATTN_ERR_ARG = 5           /* bad scalar: unknown enum value, sm_scale not finite or <= 0  */
} attn_status_t;

/*
 * attn_fwd -- enqueue O = softmax(mask(sm_scale * Q K^T)) V.
 *
 *   q, k, v, o   device pointers, contiguous [batch, heads, L, D]; element types per dtype.
 *   batch, heads, L, D
 *                sizes; batch*heads*L == 0 is a no-op that returns ATTN_OK.
 *   sm_scale     multiplies Q.K before the softmax; finite and > 0 (callers pass 1/sqrt(D)).
 *   mask_mode    an attn_mask_t value.
 *   block_size   ATTN_MASK_BLOCK_DIAG only: the diagonal block edge; must divide L
 *                ("TLX Block Attention", wrapper).  Ignored by the other modes.
 *   dtype        an attn_dtype_t value.
 *   stream       hipStream_t to enqueue on (NULL: default stream).
 *
 * Supported set (everything else returns ATTN_ERR_UNSUPPORTED):
 *   none, causal   D in {16, 32, 64, 128}: ATTN_F16, ATTN_BF16; any L >= 1 (a ragged last tile is
 *                  masked).  The page's wrapper accepts head dims 16..256 ("Fused Attention",
 *                  attention wrapper shape checks).
 *                  D = 256: ATTN_F16, ATTN_BF16, ATTN_BF16_V_E5M2, ATTN_F16_V_E5M2
 *   block_diag     D in {64, 128}: ATTN_F16, ATTN_BF16; block_size in {32, 64, 128}
 */
attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o,
                       int64_t batch, int64_t heads, int64_t L, int64_t D,
                       float sm_scale, attn_mask_t mask_mode, int64_t block_size,
                       attn_dtype_t dtype, void* stream);

/*
 * attn_fwd_lse -- attn_fwd that also writes the natural-log row normaliser
 *   lse[b, h, i] = m_i + ln(sum_j exp(S[i, j] - m_i))   (fp32, contiguous [batch, heads, L])
 * as the fused-attention page stores it for a backward pass ("Fused Attention", _attn_fwd
 * epilogue).  lse is a caller-owned device pointer; NULL behaves exactly like attn_fwd.
 */
attn_status_t attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t batch, int64_t heads, int64_t L, int64_t D,
                           float sm_scale, attn_mask_t mask_mode, int64_t block_size,
                           attn_dtype_t dtype, void* stream);

/*
 * attn_fwd_strided -- attn_fwd_lse on tensors in any layout whose last dimension (D) is contiguous,
 * such as [batch, L, heads, D] or a slice of a wider tensor.  The pages' kernels take the element
 * strides of every dimension as arguments ("TLX Block Attention", kernel arguments; "Triton-CUDA
 * Attention" and "Fused Attention", stride arguments of the kernels).
 *
 *   x_strides    host pointers to three int64 element strides of tensor x: batch, head, row
 *                (sequence position).  Element (b, h, i, d) of x sits at
 *                x + (b*x_strides[0] + h*x_strides[1] + i*x_strides[2] + d) elements.
 *   lse          as in attn_fwd_lse: NULL, or a contiguous fp32 [batch, heads, L] array.
 *
 * Requirements (else ATTN_ERR_SHAPE, nothing enqueued): strides non-negative; the row stride at
 * least D (rows of one head do not overlap); every stride, in bytes, a multiple of 16 and q, k,
 * v, o on 16-byte boundaries (lse on 4: the kernels move rows in 16-byte pieces); one head's
 * rows of one tensor span fewer than 2^31 bytes; every element offset fits int64.  o must not overlap itself, q, k or v.  A NULL
 * stride pointer returns ATTN_ERR_NULL.  attn_fwd and attn_fwd_lse are this call with the
 * contiguous strides (heads*L*D, L*D, D).
 */
attn_status_t attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t batch, int64_t heads, int64_t L, int64_t D,
                               const int64_t* q_strides, const int64_t* k_strides,
                               const int64_t* v_strides, const int64_t* o_strides, float sm_scale,
                               attn_mask_t mask_mode, int64_t block_size, attn_dtype_t dtype,
                               void* stream);

/*
 * attn_fwd_check -- run attn_fwd's host-side validation only (no HIP call, pointers may be
 * any non-NULL value).  Returns the status attn_fwd would return before launching.
 */
attn_status_t attn_fwd_check(int64_t batch, int64_t heads, int64_t L, int64_t D,
                             float sm_scale, attn_mask_t mask_mode, int64_t block_size,
                             attn_dtype_t dtype);

/* Static, NUL-terminated description of a status code ("unknown status" for others). */
const char* attn_status_str(attn_status_t status);

/* ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
