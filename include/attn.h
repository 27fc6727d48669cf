/*
 * attn.h -- C ABI of the gfx950 (MI355X) attention library (libattn_fwd.so):
 * the FlashAttention forward and backward. Plain C: no C++ types, no
 * exceptions across the boundary, no torch types. Device pointers are HIP device pointers; the
 * stream is a hipStream_t passed as void* (NULL = the default stream).
 *
 * Operation (the FlashAttention forward of "4.4 Writing GPU Kernels with
 * Triton", section "Kernel 4: A Simplified FlashAttention", whose driver
 * takes q, k, v of shape (B, H, N, d) and returns O and the per-row
 * logsumexp L): for every batch b, head h and query row i
 *
 *   s_ij   = scale * sum_c Q[b,h,i,c] K[b,h,j,c]          j in A(i)
 *   O[b,h,i,:] = sum_{j in A(i)} softmax_j(s_i.) V[b,h,j,:]
 *   LSE[b,h,i] = ln sum_{j in A(i)} exp(s_ij)             (natural log)
 *
 * where A(i) = {0, ..., N-1}, or {0, ..., i} when causal (query i sees only
 * keys j <= i -- that page's causal mask). The N x N score matrix is never
 * written to memory: the kernels stream K/V tiles and keep the online
 * softmax state (running maximum, running sum, rescaled output) on chip,
 * following that page's section "The Online Softmax Recurrence".
 */
#ifndef ATTN_FWD_ATTN_H
#define ATTN_FWD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum {
  ATTN_F32 = 0,  /* IEEE binary32 */
  ATTN_F16 = 1,  /* IEEE binary16 */
  ATTN_BF16 = 2  /* bfloat16 */
} attn_dtype;

/* Status codes. Nothing is printed and nothing aborts. */
typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,         /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,        /* B, H or N < 1, or a size beyond the limits below */
  ATTN_ERR_UNSUPPORTED = 3,  /* head dim or dtype combination not built */
  ATTN_ERR_SCALE = 4,        /* scale is NaN, infinite or negative */
  ATTN_ERR_HIP = 5,          /* the HIP runtime reported an error at launch */
  ATTN_ERR_WORKSPACE = 6,    /* a required workspace is NULL, too small or misaligned */
  ATTN_ERR_CAPACITY = 7      /* larger than the allocation-free entry point's static scratch */
} attn_status;

/* Version of this ABI (bumped on any incompatible change). */
#define ATTN_ABI_VERSION 2

/*
 * attn_fwd -- enqueue the attention forward on `stream`.
 *
 * q, k, v : device, [B][H][N][d] contiguous (row-major), element type in_dtype.
 * o       : device, [B][H][N][d] contiguous, element type out_dtype; written.
 * lse     : device, [B][H][N] contiguous fp32; written with the natural-log
 *           logsumexp of each row's scaled scores (the value the backward
 *           pass needs; "Kernel 4", notes on the saved L).
 * B, H, N : batch, heads, sequence length (queries = keys = N).
 * d       : head dimension, 64 or 128.
 * causal  : non-zero -> query i attends to keys j <= i only.
 * scale   : softmax scale, finite and >= 0; callers wanting the pages'
 *           default pass 1/sqrt(d). (A scale of exactly 0 is applied as the
 *           smallest normal fp32 number: every score then rounds to the
 *           same exponent and the weights are exactly uniform.)
 * in_dtype / out_dtype : supported pairs are
 *           (BF16, BF16) (BF16, F32) (F16, F16) (F16, F32) (F32, F32).
 *           bf16 and fp16 inputs are multiplied on the matrix cores with fp32
 *           accumulation; the softmax weights P enter the P.V product as
 *           fp16 (for bf16 inputs V is converted to fp16); softmax
 *           statistics are fp32. fp32 inputs are computed in fp32
 *           throughout.
 *           bf16 V of any finite magnitude is accepted:
 *            - |v| in [2^-14, 65504]: the fp16 copy is exact.
 *            - |v| > 65504: its fp16 copy is infinite, which makes the
 *              accumulators of the rows that meet it non-finite. The kernel
 *              checks every accumulator after the key loop and recomputes
 *              those rows with P rounded to bf16 against the bf16 V (the
 *              page's own operand precision), reading K and V from memory.
 *              Correct, but much slower for the rows concerned. The fp32
 *              accumulators bound |O| sums: max|v| * 2^8 * N must stay
 *              below fp32's range.
 *            - |v| < 2^-14: fp16's subnormal range; the copy is rounded to a
 *              multiple of 2^-24, so each output element moves by at most
 *              2^-25 (the weights of a row are non-negative and sum to 1).
 *           LSE does not depend on V and is the same in every case. Inputs
 *           holding inf or NaN give non-finite outputs.
 * stream  : hipStream_t (or NULL). The call only enqueues work and does not
 *           synchronise; a fault during execution surfaces at the caller's
 *           next synchronisation.
 *
 * Limits: N <= 2^24, B*H <= 2^24, and the launch grid ceil(N/128)*B*H must
 * fit in 2^31 - 1 workgroups; otherwise ATTN_ERR_SHAPE.
 * Ownership: the caller allocates and owns all five buffers; the library
 * allocates nothing and keeps no per-call state, so concurrent calls on
 * different streams are safe. o and lse must not alias q, k or v (not
 * checked). Buffers from a device allocator (256-byte aligned) are assumed;
 * the kernels read and write 16-byte vectors.
 * Errors: every argument is validated before any HIP call is made, so the
 * error paths need no GPU. ATTN_ERR_HIP carries the raw hipError_t in
 * attn_last_hip_error().
 */
attn_status attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                     int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                     attn_dtype in_dtype, attn_dtype out_dtype, void *stream);

/*
 * attn_fwd_workspace_bytes -- bytes of device workspace attn_fwd_ws can use
 * for this problem, 0 when it would use none.
 *
 * For bf16 inputs with N >= 8192 the bf16 -> fp16 conversion of V (see
 * in_dtype above) runs once per element in a first pass that writes an
 * fp16 copy of V, B*H*N*d*2 bytes, into the workspace, instead of once per
 * query tile inside the attention kernel. Every other problem, and
 * any invalid argument set, gives 0. No HIP call is made.
 */
size_t attn_fwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, attn_dtype in_dtype);

/*
 * attn_fwd_ws -- attn_fwd with a caller-owned device workspace.
 *
 * Arguments, validation, errors and results are those of attn_fwd; the
 * results are bitwise identical to attn_fwd's. The workspace is used only
 * when attn_fwd_workspace_bytes() > 0 for the problem, workspace_bytes is at
 * least that, and workspace is non-NULL and 16-byte aligned; otherwise it is
 * ignored and the call is exactly attn_fwd (no error is raised for it).
 * The library never allocates, frees or retains the workspace. Its contents
 * on entry do not matter and are unspecified afterwards, and it must not be
 * used by other work until the enqueued work of this call has finished on
 * `stream` (a second call on the same stream may reuse it).
 */
attn_status attn_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse,
                        int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                        attn_dtype in_dtype, attn_dtype out_dtype, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * attn_bwd_workspace_bytes -- bytes of device workspace attn_bwd needs:
 * 8 bytes per query row (B*H*N rows), rounded up to 256; 0 for an invalid
 * problem (sizes out of range, or d not a multiple of 8 in [8, 128]). No HIP
 * call is made.
 */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

/*
 * attn_bwd -- enqueue the attention backward on `stream`.
 *
 * Operation (the FlashAttention backward of "4.4 Writing GPU Kernels with
 * Triton", section "Kernel 5: FlashAttention Backward", including its
 * preprocessing step): given the forward's inputs, its output O, its
 * natural-log LSE and the upstream gradient dO, for every batch b and head h
 *
 *   P_ij  = exp(s_ij - LSE_i)      (s_ij as in attn_fwd; 0 for hidden keys)
 *   D_i   = sum_c dO_ic O_ic
 *   dS_ij = P_ij (sum_c dO_ic V_jc - D_i)
 *   dQ_i  = scale sum_j dS_ij K_j,  dK_j = scale sum_i dS_ij Q_i,
 *   dV_j  = sum_i P_ij dO_i.
 *
 * P is rebuilt tile by tile from LSE; no N x N tensor is written. The
 * preprocessing step writes (LSE * log2 e, D) per row into the workspace: for
 * bf16/fp16 inputs the query-parallel kernel that writes dQ does it for its
 * rows and runs first, for fp32 inputs a separate first pass does it; a
 * key-parallel kernel then writes dK and dV from those rows (no atomics: the
 * result is deterministic).
 *
 * q, k, v, dout : device, [B][H][N][d] contiguous, element type in_dtype
 *                 (BF16, F16 or F32).
 * o             : device, [B][H][N][d] contiguous, element type o_dtype
 *                 (in_dtype or F32; F32 for F32 inputs): the forward's output.
 * lse           : device, [B][H][N] contiguous fp32: the forward's LSE.
 * dq, dk, dv    : device, [B][H][N][d] contiguous, element type grad_dtype
 *                 (in_dtype or F32; F32 for F32 inputs); written.
 * B, H, N, causal, scale : as for attn_fwd (the forward's values).
 * d             : head dimension, a multiple of 8 in [8, 128]. The kernels
 *                 work at 64 or 128 columns; the columns past d read as
 *                 zeros (the padding note of "4.4 Writing GPU Kernels with
 *                 Triton", section "Sizing the attention kernel": a zero
 *                 column adds nothing to any score or to D, and its
 *                 gradients are zero and never stored).
 * workspace     : device, at least attn_bwd_workspace_bytes() bytes, 16-byte
 *                 aligned; caller-owned, contents on entry irrelevant and
 *                 unspecified afterwards. It must not be used by other work
 *                 until this call's work on `stream` has finished.
 * stream        : hipStream_t (or NULL); the call only enqueues work.
 *
 * Precision: Q K^T, dO V^T and the three gradient products run on the
 * matrix cores in the input type with fp32 accumulation; P and dS are
 * rounded to the input type for the products that take them, and every
 * other quantity is fp32. fp32 inputs run in fp32 throughout
 * (v_mfma_f32_32x32x2_f32), the page's check of the backward in fp32.
 * Limits and errors: those of attn_fwd, plus ATTN_ERR_WORKSPACE when the
 * workspace is NULL, too small or misaligned. Every argument is validated
 * before any HIP call. Outputs must not alias inputs (not checked).
 */
attn_status attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                     const void *dout, void *dq, void *dk, void *dv, int64_t B, int64_t H,
                     int64_t N, int64_t d, int causal, float scale, attn_dtype in_dtype,
                     attn_dtype o_dtype, attn_dtype grad_dtype, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * attn_bwd_qk -- attn_bwd with Nq query rows and Nk keys per head
 * (cross-attention). q, o, dout and dq are [B][H][Nq][d]; k, v, dk and dv
 * are [B][H][Nk][d]; lse is [B][H][Nq]. The workspace holds 8 bytes per
 * query row: attn_bwd_workspace_bytes(B, H, Nq, d). causal requires
 * Nq == Nk (else ATTN_ERR_SHAPE). Everything else is as for attn_bwd, which
 * is this call with Nq = Nk = N.
 */
attn_status attn_bwd_qk(const void *q, const void *k, const void *v, const void *o,
                        const float *lse, const void *dout, void *dq, void *dk, void *dv,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                        float scale, attn_dtype in_dtype, attn_dtype o_dtype,
                        attn_dtype grad_dtype, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * attn_bwd_strided -- attn_bwd_qk for strided tensors.
 *
 * Every tensor argument but lse comes with the element strides of its
 * (batch, head, row) dimensions, or NULL for a contiguous [B][H][n][d]
 * tensor; the column stride is 1. The kernels take the strides as they are
 * (no copies): the [B, N, H, d] layout of a fused projection, seen as
 * [B, H, N, d], needs nothing else. lse is [B][H][Nq] contiguous fp32; the
 * workspace is attn_bwd_qk's. Each view must have non-negative strides, a
 * row stride >= d, rows starting 16-byte aligned (base and every stride a
 * multiple of 16 bytes), every offset below 2^47 elements, and 128 rows
 * spanning less than 2^31 bytes; otherwise ATTN_ERR_UNSUPPORTED. The
 * inputs may share memory (a stride of 0 over heads lets H query heads read
 * one K/V head: multi- or grouped-query attention); the rows of dq, dk and
 * dv must not (ATTN_ERR_UNSUPPORTED otherwise): dK and dV are written per
 * query head, and a caller sharing K/V heads sums them over each group.
 * Every other argument, check, error and result is that of attn_bwd_qk.
 */
attn_status attn_bwd_strided(const void *q, const int64_t *q_strides, const void *k,
                             const int64_t *k_strides, const void *v, const int64_t *v_strides,
                             const void *o, const int64_t *o_strides, const float *lse,
                             const void *dout, const int64_t *dout_strides, void *dq,
                             const int64_t *dq_strides, void *dk, const int64_t *dk_strides,
                             void *dv, const int64_t *dv_strides, int64_t B, int64_t H,
                             int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                             attn_dtype in_dtype, attn_dtype o_dtype, attn_dtype grad_dtype,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_bwd_noalloc -- attn_bwd_qk without a workspace argument and without
 * any allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The 8 bytes per query row that attn_bwd_qk keeps in the caller's workspace
 * live instead in a static device array of 16 MiB inside the library (one
 * per GPU, held until the process ends), so B*H*Nq may be at most 2^21;
 * larger problems return ATTN_ERR_CAPACITY before any HIP call. The array's
 * device address is looked up (hipGetSymbolAddress) on the first call on
 * each device, which must be the current device. Nothing in it needs to
 * start at zero: every call writes each row it reads first. Calls that
 * overlap on one GPU (other streams, other threads) share the array and
 * race; serialise them. Every other argument, check, error and result is
 * that of attn_bwd_qk: the same kernels run, so the gradients are bitwise
 * the same.
 */
attn_status attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                             const float *lse, const void *dout, void *dq, void *dk, void *dv,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                             float scale, attn_dtype in_dtype, attn_dtype o_dtype,
                             attn_dtype grad_dtype, void *stream);

/*
 * attn_fwd_strided -- the attention forward of attn_fwd for general layouts:
 * Nq query rows against Nk keys per head (cross-attention; the page
 * "Programming an attention kernel in Triton", section "Kernel 4: bringing
 * it together, a self-attention kernel", checks its kernel on mismatched
 * query and key lengths), any head dimension d = 8, 16, ..., 128 (computed at 64 or 128
 * with zero-padded columns, exact by "4.4 Writing GPU Kernels with Triton",
 * section "Sizing the attention kernel"), and strided tensors.
 *
 * q          : device, element (b, h, i, c) at q + b*qs[0] + h*qs[1] + i*qs[2] + c
 *              (elements of in_dtype) for i < Nq, c < d; likewise k and v
 *              with Nk rows, and o (out_dtype) with Nq rows; written.
 * *_strides  : three int64 element strides (b, h, row), or NULL for the
 *              contiguous [B][H][n][d] layout. The column stride is 1. Each
 *              pointer and stride*element size must be a multiple of 16
 *              bytes, strides non-negative, the row stride >= d, and every
 *              offset below 2^47 elements; for bf16/fp16, 64 rows of K or V
 *              must span less than 2^31 bytes. Otherwise ATTN_ERR_UNSUPPORTED.
 *              q, k and v may share memory: a head stride of 0 lets every
 *              query head read one K/V head (multi-query attention), and q
 *              seen as [B*Hkv][G][Nq][d] with k, v as [B*Hkv][G][Nk][d] of
 *              head stride 0 gives grouped-query attention. The rows of o
 *              must not overlap (ATTN_ERR_UNSUPPORTED otherwise).
 * lse        : device, [B][H][Nq] contiguous fp32; written.
 * causal     : requires Nq == Nk (else ATTN_ERR_SHAPE).
 * d          : a multiple of 8 in [8, 128] (else ATTN_ERR_UNSUPPORTED).
 * Other arguments, dtype pairs, precision, errors and ownership are those of
 * attn_fwd. bf16/fp16 problems with row strides of at most 2^21 elements
 * run on attn_fwd's kernels (at 64 or 128 columns, those past d read as
 * zeros and not stored), reading and writing through the strides; for
 * self-attention the result equals attn_fwd's on the same values
 * zero-padded to 64 or 128 columns, bit for bit. fp32 problems (and
 * bf16/fp16 ones with longer row strides) run on a separate, simpler
 * kernel, whose results equal attn_fwd's within the forward's tolerance,
 * not bitwise.
 */
attn_status attn_fwd_strided(const void *q, const int64_t *q_strides, const void *k,
                             const int64_t *k_strides, const void *v, const int64_t *v_strides,
                             void *o, const int64_t *o_strides, float *lse, int64_t B, int64_t H,
                             int64_t Nq, int64_t Nk, int64_t d, int causal, float scale,
                             attn_dtype in_dtype, attn_dtype out_dtype, void *stream);

/*
 * attn_row_softmax -- y_ij = exp(x_ij - max_j x_ij) / sum_j exp(x_ij - max_j x_ij)
 * for every row i of an M x N matrix: the fused softmax of "4.4 Writing GPU
 * Kernels with Triton", section "Kernel 2: Fused Softmax", reading each row
 * once and writing it once (rows longer than 16384 are read twice).
 *
 * x : device, row i at x + i * x_row_stride (elements of in_dtype), N values.
 * y : device, row i at y + i * y_row_stride (elements of out_dtype); written.
 * in_dtype / out_dtype : (F32, F32), (BF16, BF16), (BF16, F32), (F16, F16),
 *     (F16, F32). Arithmetic is fp32.
 * Limits: 1 <= M < 2^31, 1 <= N <= 2^30, N <= row strides <= 2^40, pointers
 * aligned to their element size (else ATTN_ERR_SHAPE / ATTN_ERR_UNSUPPORTED).
 * Rows whose every value is -inf give NaN, as the definition does.
 * Errors, ownership and the stream: as for attn_fwd. y must not overlap x.
 */
attn_status attn_row_softmax(const void *x, int64_t x_row_stride, void *y, int64_t y_row_stride,
                             int64_t M, int64_t N, attn_dtype in_dtype, attn_dtype out_dtype,
                             void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *attn_status_string(attn_status s);

/* ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

/* Raw hipError_t behind the last ATTN_ERR_HIP returned on this thread (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_ATTN_H */
