/*
 * ptb.h -- C ABI of the MI355X (gfx950) library for one tensor-parallel shard
 * of a parallel transformer block (PTB) with causal sliding-window attention
 * (SWA), forward and backward, and the fused LAMB optimizer step.
 *
 * Sources (web pages, by title and section):
 *   [MS]  "MegaScale study guide" (ai-yanyi-papers, on arXiv:2402.15627),
 *         ch.2 §2.2 (paper §3.1), technique table: PTB row (one LayerNorm
 *         feeds both branches, y = x + MLP(LN(x)) + Attention(LN(x))), SWA row
 *         (each token attends to a fixed window w, cost O(s*w)), LAMB row
 *         (layer-wise adaptive trust ratio, You et al. 2020).
 *   [MS-T1] same page, §2.5 (paper §6.1), Table 1: 175B/530B shapes, seq 2048.
 *   [MS-TP] same page, ch.2 §2.1/§2.3: tensor parallelism splits the GEMMs of
 *         MLP and attention; each shard produces a partial sum that the
 *         collective (not part of this library) adds up.
 *
 * Conventions shared by every entry point
 *   - All device buffers are caller-owned; the library never allocates, frees
 *     or synchronizes.  Every call only enqueues kernels on `stream` (0 = the
 *     null stream) and returns; kernel faults surface at the caller's next
 *     synchronization.
 *   - Arguments are validated on the host before any launch.  A negative
 *     status means nothing was launched and no buffer was touched.
 *   - Device pointers must be 16-byte aligned.
 *   - Matrices are row-major.  Activations are token-major [T, width] with
 *     T = batch * seq and the tokens of one sequence contiguous.
 *   - Calls are reentrant.  The mutable global state is: an atomic
 *     per-process launch counter that tags the split-K arrival counters in
 *     the GEMM workspace (so workspace contents never need initialising);
 *     a per-device cache of the compute-unit count (atomic words, written
 *     once per device with the same value by any racing caller); and, for
 *     lamb_step_noalloc only, a per-device static scratch array and the
 *     cached device address of that array.
 */
#ifndef PTB_H
#define PTB_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PTB_OK = 0,
  PTB_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, misalignment   */
  PTB_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head_dim 80)    */
  PTB_ERR_WORKSPACE = -3,   /* saved/scratch buffer smaller than required      */
  PTB_ERR_HIP = -4          /* a kernel launch was rejected by the HIP runtime */
} ptb_status;

typedef enum { PTB_F32 = 0, PTB_BF16 = 1 } ptb_dtype;

/* Dimensions of one shard of the block.
 *   x, y, dy, dx : [batch*seq, hidden] in `dtype`
 *   w_in         : [3*n_heads*head_dim + ffn, hidden] in `dtype`; rows are
 *                  Q (head-major) | K | V | FC1   (the fused input GEMM of the
 *                  two branches that read the same LN(x), [MS] PTB row)
 *   w_out        : [n_heads*head_dim + ffn, hidden] in `dtype`; rows are the
 *                  attention output projection (head-major) | FC2, so
 *                  y = [x] + [O | GeLU(f)] w_out  (the two branch outputs are
 *                  summed, so their projections fuse into one GEMM)
 *   ln gamma/beta and their gradients are always fp32 [hidden].
 * Constraints: all sizes >= 1; hidden % 8 == 0, ffn % 8 == 0, hidden <= 32768;
 * head_dim in {64, 96, 128}; window >= 1, with no upper bound (any window
 * >= seq is plain causal attention and gives bit for bit the result of
 * window = seq); every matrix below 2 GiB.
 * Attention: key j is visible to query i (same sequence) iff 0 <= i-j < window
 * ([MS] SWA row), scores scaled by 1/sqrt(head_dim).  LayerNorm uses the biased
 * variance with ln_eps inside the square root.  GeLU is the exact erf form.
 * No biases, no dropout.
 * add_residual: 1 -> y = x + shard partial (rank 0 of a TP group, or TP = 1);
 *               0 -> y = shard partial only ([MS-TP]).  In backward the same
 *               flag decides whether dy is added into dx.                     */
typedef struct {
  int32_t batch, seq, hidden;
  int32_t n_heads, head_dim;
  int32_t ffn;
  int32_t window;
  int32_t add_residual;
  float ln_eps;
  int32_t dtype; /* ptb_dtype */
} ptb_dims;

/* Bytes of the `saved` buffer that ptb_forward fills and ptb_backward reads:
 * the activations only (LN output and statistics, Q|K|V, FC1
 * pre-activation, [O | GeLU(FC1)], attention log-sum-exp; for bf16 also the
 * rounding residuals of the LN output and of q, k).  175B shard, bf16:
 * about 189 MB.  0 if dims are invalid. */
size_t ptb_saved_bytes(const ptb_dims* dims);

/* Bytes of the transient `scratch` buffer (backward temporaries, and for
 * bf16 128 MiB + 32 KiB of GEMM split-K workspace that the forward uses
 * too).  One buffer serves ptb_forward and ptb_backward; nothing in it
 * outlives a call, so calls that share it must be ordered on one stream.
 * 0 if invalid. */
size_t ptb_scratch_bytes(const ptb_dims* dims);

/* Forward of one shard ([MS] PTB and SWA rows):
 *   xn = LN(x); [q|k|v|f] = xn w_in^T; O = SWA(q, k, v);
 *   y = [x] + [O | GeLU(f)] w_out.
 * Writes y and `saved` (which must stay untouched until ptb_backward).
 * scratch: ptb_scratch_bytes(dims) bytes, contents not preserved; or NULL
 * with scratch_bytes = 0, in which case every GEMM runs whole-tile
 * schedules (same results up to fp32 summation order, slower at shapes
 * whose tile count leaves compute units idle). */
int ptb_forward(const ptb_dims* dims, const void* x, const float* ln_gamma,
                const float* ln_beta, const void* w_in, const void* w_out, void* y,
                void* saved, size_t saved_bytes, void* scratch, size_t scratch_bytes,
                hipStream_t stream);

/* Backward of one shard: given dy = dL/dy, overwrites dx, d_ln_gamma,
 * d_ln_beta, dw_in, dw_out (same layouts and dtypes as their primal; the LN
 * gradients fp32).  `saved` is the buffer the matching ptb_forward filled.
 * `scratch` holds temporaries (ptb_scratch_bytes). */
int ptb_backward(const ptb_dims* dims, const void* x, const float* ln_gamma,
                 const void* w_in, const void* w_out, const void* saved,
                 size_t saved_bytes, const void* dy, void* dx, float* d_ln_gamma,
                 float* d_ln_beta, void* dw_in, void* dw_out, void* scratch,
                 size_t scratch_bytes, hipStream_t stream);

/* The serial pre-LN block that the PTB row replaces (same study guide page,
 * ch.2 §2.2 technique table, PTB row, which writes the serial form with the
 * attention residual missing; read here as the standard pre-LN layer):
 *   h = x + Attention(LN1(x));   y = h + MLP(LN2(h)).
 * Same dims, kernels and weight layout as ptb_forward (w_in rows
 * Q | K | V | FC1, w_out rows attention-out | FC2), but two LayerNorms with
 * their own fp32 (gamma, beta) and four separate projections.  LN2 needs the
 * whole h, so dims->add_residual must be 1 (else PTB_ERR_INVALID_ARG); on a
 * tensor-parallel shard this computes the shard's weights as a whole layer.
 * Buffers and errors as for ptb_forward / ptb_backward; sizes from
 * ptb_serial_saved_bytes (activations only) / ptb_serial_scratch_bytes
 * (bf16: includes the 128 MiB + 32 KiB GEMM workspace; one scratch buffer
 * serves both calls, and the forward also accepts NULL with 0 bytes).
 * Backward overwrites dx, the four LN gradients (fp32), dw_in and dw_out. */
size_t ptb_serial_saved_bytes(const ptb_dims* dims);
size_t ptb_serial_scratch_bytes(const ptb_dims* dims);
int ptb_serial_forward(const ptb_dims* dims, const void* x, const float* ln1_gamma,
                       const float* ln1_beta, const float* ln2_gamma, const float* ln2_beta,
                       const void* w_in, const void* w_out, void* y, void* saved,
                       size_t saved_bytes, void* scratch, size_t scratch_bytes,
                       hipStream_t stream);
int ptb_serial_backward(const ptb_dims* dims, const void* x, const float* ln1_gamma,
                        const float* ln2_gamma, const void* w_in, const void* w_out,
                        const void* saved, size_t saved_bytes, const void* dy, void* dx,
                        float* d_ln1_gamma, float* d_ln1_beta, float* d_ln2_gamma,
                        float* d_ln2_beta, void* dw_in, void* dw_out, void* scratch,
                        size_t scratch_bytes, hipStream_t stream);

/* One parameter tensor for lamb_step.
 *   w, m, v    fp32 device arrays of n elements, updated in place
 *   g          gradient, n elements of grad_dtype (PTB_F32 or PTB_BF16)
 *   w_bf16     optional (NULL = none): receives the updated w rounded to bf16,
 *              e.g. the low-precision weight the next forward reads
 *   weight_decay  this tensor's decoupled weight decay                      */
typedef struct {
  float* w;
  const void* g;
  float* m;
  float* v;
  void* w_bf16;
  int64_t n;
  float weight_decay;
  int32_t grad_dtype;
} lamb_tensor;

/* Bytes of the scratch buffer lamb_step needs for these tensors (block
 * partial sums of ||w||^2 and ||u||^2 and the per-tensor ratios). */
size_t lamb_scratch_bytes(const lamb_tensor* tensors, int32_t n_tensors);

/* One LAMB step ([MS] LAMB row; the method of You et al. 2020) over every
 * tensor, each tensor being one "layer" of the trust ratio:
 *   m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
 *   u = (m / (1-b1^step)) / (sqrt(v / (1-b2^step)) + eps) + weight_decay * w;
 *   r = ||w|| / ||u||  (r = 1 if either norm is 0);  w <- w - lr * r * u.
 * `tensors` is a HOST array of n_tensors descriptors (device pointers inside);
 * step >= 1; 0 <= beta < 1; eps > 0 and finite (with eps = 0 a zero gradient
 * on zero moments would make u = 0/0, so it is rejected as
 * PTB_ERR_INVALID_ARG).  ratios_out: optional device float[n_tensors]
 * receiving r.  The norms are exact two-pass reductions: pass A writes m, v
 * and per-workgroup partial sums, a finalize kernel adds them in fp64 in a
 * fixed order (deterministic), pass B recomputes u and applies w. */
int lamb_step(const lamb_tensor* tensors, int32_t n_tensors, float lr, float beta1, float beta2,
              float eps, int64_t step, float* ratios_out, void* scratch, size_t scratch_bytes,
              hipStream_t stream);

/* Sharded LAMB for data-parallel training with ZeRO-2 optimizer sharding
 * (MegaScale study guide, ch.2 §2.1 parallelism table, DP (+ZeRO-2) row:
 * optimizer state and gradients are split over the data-parallel ranks;
 * the trust ratio as in lamb_step): every rank owns a contiguous element range of each
 * tensor, and the descriptors passed here point at this rank's range (n =
 * its length; any split works, the step is elementwise apart from the two
 * norms).  The step splits at the norms:
 *   lamb_shard_norms  updates m and v of the shard in place exactly as
 *                     lamb_step does and writes norms_out[2 t] = sum of w^2
 *                     and norms_out[2 t + 1] = sum of u^2 over the shard
 *                     (device fp64 [2 n_tensors], 8-byte aligned);
 *   (caller)          sums norms_out over the ranks, e.g. an all-reduce of
 *                     2 n_tensors doubles, into `norms`;
 *   lamb_shard_apply  r_t = sqrt(norms[2t]) / sqrt(norms[2t+1]) (1 if either
 *                     is 0), then w <- w - lr * r_t * u on the shard (and
 *                     w_bf16 if given); g may be NULL here.
 * With one shard per tensor this is lamb_step; across shards the results
 * differ from it only by the order of the fp64 norm sums.  Same scratch
 * size and rules as lamb_step (lamb_scratch_bytes of the shard
 * descriptors); the two halves must see the same hyper-parameters and
 * step.  Errors as lamb_step. */
int lamb_shard_norms(const lamb_tensor* tensors, int32_t n_tensors, float beta1, float beta2,
                     float eps, int64_t step, double* norms_out, void* scratch,
                     size_t scratch_bytes, hipStream_t stream);
int lamb_shard_apply(const lamb_tensor* tensors, int32_t n_tensors, float lr, float beta1,
                     float beta2, float eps, int64_t step, const double* norms,
                     float* ratios_out, void* scratch, size_t scratch_bytes, hipStream_t stream);

/* lamb_step for callers that cannot allocate device memory (code under
 * graph capture, tight loops, harnesses that forbid allocation): the same
 * step, kernels and results as lamb_step, with the scratch taken from a
 * static array in device memory (one per device, kept until the process
 * ends) instead of a caller buffer.  It calls no allocating routine.
 * Limit: lamb_scratch_bytes(tensors, n_tensors) must not exceed
 * lamb_noalloc_max_scratch_bytes() (2 MiB: about 1.07e9 parameters split
 * over few tensors), else PTB_ERR_WORKSPACE and nothing runs.  The stream
 * must belong to the current device (else PTB_ERR_INVALID_ARG); the first
 * call on a device looks up that device's copy of the array (PTB_ERR_HIP if
 * the lookup fails).  Every call on one device shares that device's array:
 * calls that overlap on one device (several streams or threads) race, so the
 * caller orders them.  Other arguments and errors as lamb_step. */
size_t lamb_noalloc_max_scratch_bytes(void);
int lamb_step_noalloc(const lamb_tensor* tensors, int32_t n_tensors, float lr, float beta1,
                      float beta2, float eps, int64_t step, float* ratios_out,
                      hipStream_t stream);

/* Human-readable text of a status code (static string). */
const char* ptb_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* PTB_H */
