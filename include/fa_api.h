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
 *   Threads    Reentrant; fa_last_error() is per host thread.  Two entry
 *              points keep state: fa_fwd_splitkv_noalloc shares one scratch
 *              array per GPU between its calls (overlapping calls race), and
 *              fa_softmax_set_wait_limit sets a process-wide bound.
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
 * FP8 fused forward: fa_fwd's result for inputs held as 8-bit floats.
 *
 * Section "4. 减少访存的几种办法" of the xinc.fun archive 235 page lets the
 * matrix products run on FP8 operands while accumulation, softmax and
 * normalisation keep a wider format; this entry point does that with the
 * online-softmax recurrence of fa_fwd.  Q, K, V hold OCP FP8 E4M3 codes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite
 * value 448; codes 0x7F and 0xFF are NaN) and each tensor has one fp32
 * scale: element x of Q stands for q_scale * e4m3(x), likewise K and V.
 * The result is
 *     O   = softmax(scale * (q_scale Q)(k_scale K)^T) (v_scale V)
 *     LSE = ln sum_j exp(scale * q_scale * k_scale * q_i . k_j)
 * with the scores accumulated in fp32 from exact code products, the
 * softmax in fp32, the probabilities rounded to E4M3 (nearest-even) for the
 * P V product with fp32 accumulation, and O rounded to bf16 (nearest-even).
 *
 *   Q, K, V  in:  (B, H, N, d) E4M3 codes (one byte each), 16-byte aligned,
 *                 finite codes only.
 *   O        out: (B, H, N, d) bf16, 16-byte aligned; must not overlap
 *                 Q, K, V or LSE.
 *   LSE      out: (B, H, N) fp32, 4-byte aligned, required; must not
 *                 overlap Q, K, V or O.
 *   scale    finite fp32 multiplier of the scores (1/sqrt(d) usually).
 *   q_scale, k_scale, v_scale
 *            finite and > 0 (FA_ERR_SCALE otherwise); |scale| * q_scale *
 *            k_scale must also be finite in fp32.
 * Other conventions (shapes, limits, stream, errors) as fa_fwd.
 */
int fa_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE,
               int64_t B, int64_t H, int64_t N, int64_t d, float scale,
               float q_scale, float k_scale, float v_scale, void* stream);

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

/*
 * Split-KV forward: the same result as fa_fwd, computed in two passes so
 * that problems with few query tiles (small B * H * N) still fill the chip.
 *   pass 1  the keys are cut into G contiguous ranges of whole key tiles;
 *           every (head, key range, query tile) is one workgroup of the
 *           fused kernel, writing its normalised partial output O_g (fp32)
 *           and log-sum-exp LSE_g for its range only;
 *   pass 2  fa_merge_partials' kernel combines the G partials per row.
 * The combination is the block merge of the special-jiahao.github.io
 * "Flash Attention" note, section "增量求解 softmax" (the global softmax
 * from the blocks' local ones), for G blocks: LSE = ln sum_g e^{LSE_g},
 * O = sum_g e^{LSE_g - LSE} O_g.
 *
 *   num_splits  G requested; 0 (or less) chooses G so that pass 1 has about
 *               2048 waves (eight per CU) while every range keeps at least
 *               1024 keys; G is clamped to [1, min(64, key tiles)].
 *               With G = 1 the call is fa_fwd and the workspace is unused.
 *   workspace   caller-owned device memory of at least
 *               fa_splitkv_workspace_bytes(B, H, N, d, dtype, num_splits)
 *               bytes, 16-byte aligned, not overlapping any argument; may be
 *               NULL when that size is 0.  Contents on return: the partials
 *               (G x B*H*N*d fp32 outputs, then G x B*H*N fp32 LSEs).
 *   workspace_bytes  its size; a smaller size than needed is FA_ERR_SHAPE.
 * Other arguments, layouts and errors as fa_fwd.
 */
int fa_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   void* workspace, size_t workspace_bytes, int num_splits, int64_t B,
                   int64_t H, int64_t N, int64_t d, float scale, int dtype, void* stream);

/*
 * fa_fwd_splitkv without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid the allocator.  The partials go to a scratch
 * array the library itself holds, FA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU
 * it runs on, in place from that device's first such call until the
 * process ends.  The call allocates nothing and frees nothing.
 *   num_splits  as fa_fwd_splitkv.  If the resolved G needs more than
 *               FA_NOALLOC_SCRATCH_BYTES (fa_splitkv_workspace_bytes() tells
 *               how much), the call returns FA_ERR_SHAPE and enqueues
 *               nothing; num_splits = 1 needs no scratch at all.
 * The scratch used is that of the calling thread's current device, and
 * `stream` must belong to that device.  Every call on one GPU shares that
 * GPU's array and leaves its partials there; nothing in it needs to start
 * at zero.  Calls that overlap on one GPU (concurrent streams, or threads
 * without ordering between their streams) race on the array and may return
 * wrong results: order them.  Other arguments, results and errors as
 * fa_fwd_splitkv; FA_ERR_HIP if the array's address cannot be obtained.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fa_fwd_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                           int num_splits, int64_t B, int64_t H, int64_t N, int64_t d,
                           float scale, int dtype, void* stream);

/* The G that fa_fwd_splitkv uses for `requested` (see above); 0 for invalid
 * sizes (including sizes beyond the limits above) or dtype. */
int fa_splitkv_num_splits(int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int requested);

/* Workspace bytes fa_fwd_splitkv needs: G * B*H*N * (d + 1) * 4 for the G it
 * resolves, 0 when G = 1 or for invalid arguments. */
size_t fa_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype,
                                  int num_splits);

/*
 * Split-KV forward for queries and keys of different lengths: Q and O are
 * (B, H, Nq, d), K and V (B, H, Nk, d), LSE (B, H, Nq); every query row
 * attends to all Nk key rows of its head.  It serves decode (a few query
 * rows, often one, against a long key sequence: the case the key-range split
 * exists for, since the query tiles alone give the chip almost no
 * workgroups) and attention of one sequence over another.  The definition is
 * that of fa_fwd with S = scale * Q K^T of shape Nq x Nk; the two passes are
 * those of fa_fwd_splitkv, with G chosen from the query tiles (for the waves
 * of pass 1) and the key tiles (for the range lengths).
 *   num_splits  as fa_fwd_splitkv, except that with fewer than 128 query
 *               rows per head (one query tile: decode) the automatic G aims
 *               at about 1024 waves, one 4-wave workgroup per CU, since each
 *               workgroup is then bound by its stream of keys and values;
 *               each key range then keeps at least 128 keys, and more than
 *               16 ranges are taken only while each keeps 512.
 *   Nq = 0 (or B = 0 or H = 0) is an empty call; Nq > 0 with Nk = 0 is
 *   FA_ERR_SHAPE (a softmax over no keys is undefined).  Both lengths obey
 *   the limits of fa_fwd.  fa_fwd_splitkv(..., N, ...) is this call with
 *   Nq = Nk = N.  Other arguments, workspace, results and errors as
 *   fa_fwd_splitkv, with B*H*Nq rows of partials.
 */
int fa_fwd_splitkv_qk(const void* Q, const void* K, const void* V, void* O, float* LSE,
                      void* workspace, size_t workspace_bytes, int num_splits, int64_t B,
                      int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int dtype,
                      void* stream);

/* The G that fa_fwd_splitkv_qk uses for `requested`; 0 for invalid sizes or
 * dtype (including Nq or Nk below 1). */
int fa_splitkv_qk_num_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int dtype,
                             int requested);

/* Workspace bytes fa_fwd_splitkv_qk needs: G * B*H*Nq * (d + 1) * 4 for the
 * G it resolves, 0 when G = 1 or for invalid arguments. */
size_t fa_splitkv_qk_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                     int dtype, int num_splits);

/*
 * Merge of num_parts partial attention results over disjoint key sets (the
 * block merge of the special-jiahao.github.io "Flash Attention" note,
 * section "增量求解 softmax", for num_parts blocks), per row r:
 *     LSE[r] = ln sum_g e^{LSE_part[g][r]}
 *     O[r]   = sum_g e^{LSE_part[g][r] - LSE[r]} O_part[g][r]
 * It is the combining step of fa_fwd_splitkv, and the step a caller would
 * run after gathering per-device partials of a key-sharded attention.
 *   O_part    in:  (num_parts, rows, d) fp32, each row normalised by its own
 *                  block's denominator; 16-byte aligned.
 *   LSE_part  in:  (num_parts, rows) fp32 natural-log log-sum-exps; -inf
 *                  marks a block without keys (its O_part row is ignored
 *                  but must be finite); 4-byte aligned.
 *   O         out: (rows, d) in `dtype` (RNE), 16-byte aligned.
 *   LSE       out: (rows) fp32, 4-byte aligned; -inf (and O = 0) for a row
 *                  whose blocks are all empty.
 *   num_parts 1 .. 4096; rows >= 0 (0: nothing is enqueued); d in {64, 128}.
 * Outputs must not overlap inputs.  Errors as fa_fwd.
 */
int fa_merge_partials(const float* O_part, const float* LSE_part, int num_parts, int64_t rows,
                      int64_t d, void* O, float* LSE, int dtype, void* stream);

/*
 * Row softmax Y[r, :] = e^{X[r, :] - m_r} / l_r with m_r the row maximum and
 * l_r = sum_j e^{X[r, j] - m_r}; LSE[r] = m_r + ln l_r.  The online softmax
 * of xinc.fun archive 235, section "7. Online Softmax" (a running maximum and
 * denominator, the old denominator rescaled by e^{m_old - m_new} when a
 * block raises the maximum), as a memory-bound operation of its own.  Rows
 * are cut into pieces whose (m, l) pairs are combined with the block merge
 * of the special-jiahao.github.io "Flash Attention" note ("增量求解 softmax"):
 *   rows of at most 8192 (16-bit) / 4096 (fp32) elements: one workgroup per
 *     row; X read once, Y written once;
 *   rows of at most 32 slices of 16384 (16-bit) / 8192 (fp32) elements whose
 *     length keeps them 16-byte aligned, with X and Y 16-byte aligned: one
 *     workgroup per slice holds it in registers until the row's pairs are
 *     merged (X read once), provided the device can hold that many
 *     workgroups at once;
 *   other rows: the pairs of 8192 / 4096-element chunks are merged per row
 *     between two passes (X read twice).
 * The three-pass maximum / sum / normalise form reads X three times;
 * fa_softmax_x_reads() tells which form a call takes.
 *   X    in:  (rows, n) contiguous, `dtype`, element-aligned (rows of a
 *             length that keeps them 16-byte aligned use 16-byte accesses).
 *   Y    out: (rows, n) contiguous, `dtype` (RNE); may equal X (in place),
 *             must not otherwise overlap it.
 *   LSE  out: (rows) fp32, or NULL.
 *   workspace  caller-owned device memory of fa_softmax_workspace_bytes()
 *             bytes, 8-byte aligned; NULL allowed when that size is 0.  Its
 *             contents need no initialisation; calls sharing one workspace
 *             must be ordered (one stream, or synchronised streams).
 * Arithmetic is fp32 for every dtype.  The one-pass slice form waits inside
 * a kernel for the other slices of a row; each wait is bounded, and slices
 * whose wait ran out are written by a further kernel of the same call, so
 * the result never depends on how many workgroups ran at once.  rows or n
 * equal to 0: nothing is enqueued.  Errors as fa_fwd.
 */
int fa_softmax_rows(const void* X, void* Y, float* LSE, int64_t rows, int64_t n, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fa_softmax_rows needs: for rows longer than one chunk the
 * larger of rows * (chunks + 1) * 8 (two passes: chunk pairs and row pairs)
 * and 16 + 12 * rows * slices (one pass: counters, slice pairs and flags),
 * else 0 (also for invalid arguments and sizes that do not fit size_t). */
size_t fa_softmax_workspace_bytes(int64_t rows, int64_t n, int dtype);

/* How many times fa_softmax_rows with these arguments would read X from
 * memory on the current device: 1 (one-chunk rows, slice-resident rows) or
 * 2 (two passes); 0 for invalid arguments.  X and Y only matter through
 * their 16-byte alignment; nothing is dereferenced or enqueued. */
int fa_softmax_x_reads(const void* X, const void* Y, int64_t rows, int64_t n, int dtype);

/* Diagnostics: sets the number of polls after which a slice of the one-pass
 * form stops waiting for the rest of its row and leaves itself to the repair
 * kernel (default 400, about half a millisecond; 0 gives up after one poll,
 * which exercises the repair path; negative restores the default).  Returns
 * the previous setting.  Process-wide; results do not depend on it. */
int fa_softmax_set_wait_limit(int polls);

/*
 * Backward pass of exact attention: dQ, dK, dV for an upstream gradient dO
 * of O = softmax(scale * Q K^T) V, from Q, K, V, the forward's O and LSE.
 * As xinc.fun archive 235, section "7. Online Softmax", closes: the scores
 * are recomputed tile by tile from the saved inputs and the log-sum-exp,
 * never read from a stored attention matrix:
 *     P = exp(scale * Q K^T - LSE),   D = rowsum(dO * O),
 *     dS = P * (dO V^T - D),   dV = P^T dO,
 *     dQ = scale * dS K,   dK = scale * dS^T Q.
 * 16-bit inputs only (FA_F16, FA_BF16; FA_F32 is FA_ERR_DTYPE): products on
 * MFMA with fp32 accumulation, P and dS rounded to the input type for the
 * products, outputs rounded (RNE) to the input type.  Deterministic (no
 * atomics): dQ and dK/dV are computed by separate kernels, each recomputing
 * the scores it needs.
 *   Q, K, V, O, dO  in:  (B, H, N, d) `dtype`, 16-byte aligned; O and LSE as
 *                        fa_fwd wrote them (for these Q, K, V and scale).
 *   LSE             in:  (B, H, N) fp32.
 *   dQ, dK, dV      out: (B, H, N, d) `dtype`, 16-byte aligned, overlapping
 *                        no input, each other or the workspace.
 *   workspace       caller-owned, fa_bwd_workspace_bytes(B, H, N) bytes,
 *                   16-byte aligned; holds (LSE * log2 e, -D) per row on return,
 *                   D = rowsum(dO * O).
 * Other arguments and errors as fa_fwd.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* LSE, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
           int64_t B, int64_t H, int64_t N, int64_t d, float scale, int dtype, void* stream);

/* Workspace bytes of fa_bwd: B * H * N * 8 (0 for negative sizes or a
 * size that does not fit size_t). */
size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N);

/* Bytes of ONE naive workspace (S or P): B * H * N * ldS * sizeof(dtype),
 * ldS = N rounded up to a multiple of 8.  Returns 0 for an invalid dtype,
 * negative sizes, N above the naive path's limit (32768) or a size that does
 * not fit size_t. */
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
