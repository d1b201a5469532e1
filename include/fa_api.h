/*
 * fa_api.h -- C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * The operation is standard attention as defined in section
 * "6. 标准注意力为什么慢" of the xinc.fun archive 235 page:
 *     S = scale * Q K^T,   P = Softmax(S) (row-wise),   O = P V
 * with scale = 1/sqrt(d) on that page; here it is a caller argument.  The
 * fused entry point computes it tile by tile with the online-softmax
 * recurrence of section "7. Online Softmax" of the same page (running row
 * maximum m, denominator l and un-normalised output, rescaled by
 * e^{m_old - m_new} when the maximum grows), so S and P never reach device
 * memory; the naive entry point runs the three steps as three kernels with S
 * and P stored in device memory, the access pattern that section
 * "MAC分析 / 标准Transformer MAC分析" of the ctyun.cn FlashAttention article
 * counts (4Nd + 4N^2 elements per head).
 *
 * Common conventions for every entry point:
 *   Layout     Q, K, V, O: contiguous (B, H, N, d) row-major, d fastest, all
 *              in the same element type `dtype`.  Head (b, h) starts at
 *              element ((b * H + h) * N) * d.  LSE: contiguous (B, H, N) fp32.
 *   Ownership  Every pointer is device memory owned by the caller.  The
 *              library never allocates, frees or synchronises and keeps no
 *              pointer after a call returns.
 *   Stream     `stream` is a hipStream_t (NULL = the default stream).  Work is
 *              enqueued asynchronously on it; the call returns before the GPU
 *              finishes.  Faults during execution surface at the caller's
 *              next synchronisation on that stream.
 *   Errors     Arguments are validated before anything is enqueued.  On a
 *              bad argument the call returns a non-zero fa_status, enqueues
 *              nothing and records a message for fa_last_error().  A failed
 *              kernel launch returns FA_ERR_HIP.
 *   Empty      B, H or N equal to 0 is a valid empty problem: FA_OK, nothing
 *              is enqueued, and pointers may then be NULL.
 *   Limits     d in {64, 128}; N * d < 2^31; B * H < 2^31; the number of
 *              workgroups < 2^31.  Values are not checked for NaN/Inf.
 *   Threads    Stateless and reentrant; fa_last_error() is per host thread.
 */
#ifndef IOFA_FA_API_H
#define IOFA_FA_API_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V, O (and of the naive path's S and P). */
typedef enum {
  FA_F32 = 0,  /* IEEE binary32; products and sums in fp32 */
  FA_F16 = 1,  /* IEEE binary16; MFMA products, fp32 accumulation/softmax */
  FA_BF16 = 2  /* bfloat16; MFMA products, fp32 accumulation/softmax */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,     /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,    /* negative or too large B, H, N */
  FA_ERR_HEAD_DIM = 3, /* d not in {64, 128} */
  FA_ERR_DTYPE = 4,    /* dtype not an fa_dtype value */
  FA_ERR_ALIGN = 5,    /* Q, K, V, O, S, P not 16-byte aligned, or LSE not 4-byte */
  FA_ERR_SCALE = 6,    /* scale is NaN or infinite */
  FA_ERR_ALIAS = 7,    /* an output overlaps an input or another output */
  FA_ERR_HIP = 8       /* the HIP runtime reported an error (see fa_last_error) */
} fa_status;

/*
 * Fused forward (FlashAttention): O = softmax(scale * Q K^T) V and
 * LSE[b,h,i] = ln sum_j exp(scale * q_i . k_j).
 *
 * Per workgroup a tile of query rows stays on chip while tiles of K and V
 * stream through LDS; scores and probabilities live only in registers
 * (xinc.fun archive 235, "6. 标准注意力为什么慢" and "7. Online Softmax";
 * ctyun.cn FlashAttention article, "核心思想").  16-bit inputs use bf16/fp16
 * MFMA products with fp32 accumulation; the probabilities are rounded to the
 * input type (nearest-even) for the P V product; the row sums and the output
 * accumulator stay fp32; O is rounded to the input type (nearest-even).
 * LSE is the natural-log log-sum-exp of the scaled scores, the statistic a
 * backward pass keeps.
 *
 *   Q, K, V  in:  (B, H, N, d) `dtype`, 16-byte aligned.
 *   O        out: (B, H, N, d) `dtype`, 16-byte aligned; must not overlap
 *                 Q, K, V or LSE.
 *   LSE      out: (B, H, N) fp32, 4-byte aligned, required (not NULL); must
 *                 not overlap Q, K, V or O.
 *   scale    finite fp32 multiplier of Q K^T (1/sqrt(d) for the usual case).
 *   dtype    an fa_dtype value.
 * Returns FA_OK or an fa_status.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
           int64_t B, int64_t H, int64_t N, int64_t d, float scale, int dtype,
           void* stream);

/*
 * Naive three-kernel forward, kept as the measured contrast of the ctyun.cn
 * article's "MAC分析 / 标准Transformer MAC分析" (and of the three-step
 * listing in section "Standard Attention" of the special-jiahao.github.io
 * "Flash Attention" note):
 *   kernel 1 reads Q, K and writes S = scale * Q K^T to S_ws (in `dtype`);
 *   kernel 2 reads S row by row and writes P = softmax(S) to P_ws
 *            (in `dtype`) and, if LSE is not NULL, the row log-sum-exp;
 *   kernel 3 reads P, V and writes O = P V.
 * S_ws and P_ws are caller-owned workspaces of fa_naive_workspace_bytes()
 * bytes each, 16-byte aligned, laid out (B, H, N, ldS) with
 * ldS = N rounded up to a multiple of 8; P's padding columns are written
 * as zeros.  N is limited to 32768 (a row of S is held in registers).
 *
 *   LSE may be NULL (then it is not written).  Other arguments as fa_fwd.
 *   S_ws, P_ws must not overlap each other, the inputs or the outputs.
 */
int fa_naive_fwd(const void* Q, const void* K, const void* V, void* O,
                 float* LSE, void* S_ws, void* P_ws, int64_t B, int64_t H,
                 int64_t N, int64_t d, float scale, int dtype, void* stream);

/* Bytes of ONE naive workspace (S or P): B * H * N * ldS * sizeof(dtype),
 * ldS = N rounded up to a multiple of 8.  Returns 0 for an invalid dtype
 * or negative sizes. */
size_t fa_naive_workspace_bytes(int64_t B, int64_t H, int64_t N, int dtype);

/* Static English text for an fa_status value ("unknown status" otherwise). */
const char* fa_status_string(int status);

/* Detail of the last failure on the calling host thread ("" if none).  The
 * pointer stays valid until the next library call on this thread. */
const char* fa_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IOFA_FA_API_H */
