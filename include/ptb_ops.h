/*
 * ptb_ops.h -- the individual steps of the block as separate C entry points.
 *
 * ptb_forward/ptb_backward (ptb.h) chain these same kernels.  They are
 * exported so that each step can be checked on its own and so that other
 * block arrangements (for instance the serial pre-LN block that the parallel
 * block replaces, MegaScale study guide ch.2 §2.2, PTB row) can be assembled
 * from them.  Conventions (ownership, stream, validation, alignment, error
 * codes) are those of ptb.h.
 */
#ifndef PTB_OPS_H
#define PTB_OPS_H

#include "ptb.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Stages of ptb_forward, in order.  ptb_forward runs all of them; each is one
 * kernel launch.                                                             */
enum {
  PTB_FWD_LAYERNORM = 0, /* xn, mean, rstd = LN(x)                    (PTB row) */
  PTB_FWD_GEMM_IN = 1,   /* [q|k|v|f] = xn w_in^T; cat[:, A:] = GeLU(f)        */
  PTB_FWD_ATTENTION = 2, /* cat[:, :A] = SWA(q, k, v); lse          (SWA row) */
  PTB_FWD_GEMM_OUT = 3,  /* y = [x] + cat w_out                                */
  PTB_FWD_STAGES = 4
};
/* Stages of ptb_backward, in order (each one to three kernel launches).    */
enum {
  PTB_BWD_GEMM_DCAT = 0,   /* dcat = dy w_out^T; dO and dz[:, 3A:] = dg GeLU'(f) */
  PTB_BWD_GEMM_DW_OUT = 1, /* dw_out = cat^T dy                                 */
  PTB_BWD_ATTENTION = 2,   /* D = rowsum(dO O); dK, dV; dQ -> dz[:, :3A]        */
  PTB_BWD_GEMM_DW_IN = 3,  /* dw_in = dz^T xn                                   */
  PTB_BWD_GEMM_DXN = 4,    /* dxn = dz w_in (temporary in the layer dtype)      */
  PTB_BWD_LAYERNORM = 5,   /* dx = LN'(dxn) [+ dy]; dgamma, dbeta               */
  PTB_BWD_STAGES = 6
};

/* One stage of ptb_forward / ptb_backward, with the same arguments, buffers,
 * validation and errors as the full call (stage -1 = every stage, which is
 * what ptb_forward and ptb_backward do).  Running the stages 0..N-1 in order
 * on one stream is exactly the full call; a stage reads what the earlier
 * stages wrote into `saved` / `scratch`. */
int ptb_forward_stage(const ptb_dims* dims, int32_t stage, const void* x, const float* ln_gamma,
                      const float* ln_beta, const void* w_in, const void* w_out, void* y,
                      void* saved, size_t saved_bytes, void* scratch, size_t scratch_bytes,
                      hipStream_t stream);
int ptb_backward_stage(const ptb_dims* dims, int32_t stage, const void* x, const float* ln_gamma,
                       const void* w_in, const void* w_out, const void* saved, size_t saved_bytes,
                       const void* dy, void* dx, float* d_ln_gamma, float* d_ln_beta, void* dw_in,
                       void* dw_out, void* scratch, size_t scratch_bytes, hipStream_t stream);

/* LayerNorm over each row of x [rows, width] (the shared pre-LN of the PTB
 * row): xn = (x - mean) / sqrt(var + eps) * gamma + beta, biased variance.
 * x and xn in `dtype`; gamma, beta [width] fp32; mean, rstd [rows] fp32
 * receive each row's mean and 1/sqrt(var + eps).  width % 8 == 0,
 * width <= 32768. */
int ptb_layernorm_forward(int32_t dtype, int32_t rows, int32_t width, const void* x,
                          const float* gamma, const float* beta, float eps, void* xn,
                          float* mean, float* rstd, hipStream_t stream);

/* Backward of ptb_layernorm_forward for the same x, gamma and the mean, rstd
 * it wrote: given dxn [rows, width] in `dtype`, writes
 *   dx = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat)) [+ dy]
 * with xhat = (x - mean) * rstd and dxhat = dxn * gamma, in `dtype` (dy:
 * optional residual gradient [rows, width] in `dtype`, NULL = none), and
 * overwrites dgamma = sum over rows of dxn * xhat and dbeta = sum over rows
 * of dxn (fp32 [width]); the column sums are added in a fixed order, so the
 * result is deterministic.  scratch: ptb_layernorm_scratch_bytes(rows,
 * width) bytes of per-workgroup partial sums, contents not preserved.
 * width % 8 == 0, width <= 32768. */
size_t ptb_layernorm_scratch_bytes(int32_t rows, int32_t width);
int ptb_layernorm_backward(int32_t dtype, int32_t rows, int32_t width, const void* x,
                           const float* gamma, const float* mean, const float* rstd,
                           const void* dxn, const void* dy, void* dx, float* dgamma,
                           float* dbeta, void* scratch, size_t scratch_bytes,
                           hipStream_t stream);

/* The GEMM engine: C[m, n] = sum_k A(m, k) * B(n, k), for m < M, n < N.
 *   a_layout 0: A(m, k) = a[m*lda + k]      1: A(m, k) = a[k*lda + m]
 *   b_layout 0: B(n, k) = b[n*ldb + k]      1: B(n, k) = b[k*ldb + n]
 *   C row-major with leading dimension ldc, in `dtype`, or fp32 when c_f32.
 * bf16: the contiguous dimension of each operand and lda, ldb, ldc must be
 * multiples of 8, and each operand below 2 GiB.  fp32 operands give fp32 C.
 * workspace (bf16 only, may be NULL; device memory, 256-byte aligned, at
 * least ptb_gemm_workspace_bytes(), owned by the caller, contents need not
 * be initialised): with it, shapes whose tile count leaves CUs idle are
 * split along K across all CUs (stream-K) and the partial tiles are summed
 * in a fixed order, so results stay deterministic.  Calls that share a
 * workspace must be ordered on one stream.  A workspace that is too small or
 * misaligned gives PTB_ERR_WORKSPACE. */
size_t ptb_gemm_workspace_bytes(void);
int ptb_gemm(int32_t dtype, int32_t a_layout, int32_t b_layout, int32_t M, int32_t N, int32_t K,
             const void* a, int64_t lda, const void* b, int64_t ldb, void* c, int64_t ldc,
             int32_t c_f32, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Sliding-window attention forward (SWA row: key j visible to query i iff
 * 0 <= i - j < window; scale 1/sqrt(head_dim)).  qkv [batch*seq, 3*H*d] in
 * dims->dtype (q | k | v, each head-major); o receives [batch*seq, H*d] with
 * leading dimension ldo; lse fp32 [batch, H, seq] receives the natural
 * log-sum-exp of each query's scaled visible scores.  Only the dims fields
 * batch, seq, n_heads, head_dim, window, dtype matter (the others must still
 * be valid). */
int ptb_swa_forward(const ptb_dims* dims, const void* qkv, void* o, int64_t ldo, float* lse,
                    hipStream_t stream);

/* Its backward: given o and lse from ptb_swa_forward and d_o [batch*seq, H*d]
 * (leading dimension H*d), writes dq | dk | dv into dqkv [batch*seq, 3*H*d].
 * dvec: fp32 [batch, H, seq] temporary. */
int ptb_swa_backward(const ptb_dims* dims, const void* qkv, const void* o, int64_t ldo,
                     const void* d_o, const float* lse, void* dqkv, float* dvec,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* PTB_OPS_H */
