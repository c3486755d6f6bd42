// Internal launchers shared between the kernel files and the C-ABI layer.
// Every launcher only enqueues work on `stream` and returns the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptb {

// Operand layouts of the GEMM engine C[m, n] = sum_k A(m, k) * B(n, k):
//   kKContig : A(m, k) = A[m * lda + k]   (B(n, k) = B[n * ldb + k])
//   kMNContig: A(m, k) = A[k * lda + m]   (B(n, k) = B[k * ldb + n])
enum Layout { kKContig = 0, kMNContig = 1 };

struct GemmDesc {
  int M, N, K;
  int a_layout, b_layout;
  const void* a;
  int64_t lda;
  const void* b;
  int64_t ldb;
  // bf16 only: tiles whose first column is below n_split add a second K pass
  // over a2 (same layout as a), i.e. C = (A + A2) B^T there.
  const void* a2 = nullptr;
  int n_split = 0;
  // bf16 only: workspace for split (stream-K) schedules; may be null, then
  // every workgroup computes whole tiles.  Needs kGemmWsBytes.
  void* ws = nullptr;
  size_t ws_bytes = 0;
};
// Stream-K: at most kSkMaxGrid persistent workgroups, each with two fp32
// 256 x 256 partial tiles in the workspace, followed by one 8-byte arrival
// counter per split tile (at most kSkMaxSplitTiles).
constexpr int kSkMaxGrid = 256;
constexpr int kSkMaxSplitTiles = 4096;
constexpr size_t kGemmPartialBytes = (size_t)2 * kSkMaxGrid * 256 * 256 * 4;
constexpr size_t kGemmWsBytes = kGemmPartialBytes + (size_t)kSkMaxSplitTiles * 8;

// ---- layernorm.hip
// xn_lo (bf16 only, may be null): receives xn - bf16(xn) rounded to bf16.
hipError_t launch_ln_fwd(int dtype, const void* x, const float* gamma, const float* beta,
                         float eps, int rows, int width, void* xn, void* xn_lo, float* mean,
                         float* rstd, hipStream_t s);
int ln_bwd_rows_per_block();
// dxn in the activation dtype.
hipError_t launch_ln_bwd(int dtype, const void* x, const float* gamma, const float* mean,
                         const float* rstd, const void* dxn, const void* dy_residual, void* dx,
                         float* gpart, float* bpart, int rows, int width, hipStream_t s);
hipError_t launch_ln_bwd_reduce(const float* gpart, const float* bpart, int nblk, int width,
                                float* dgamma, float* dbeta, hipStream_t s);

// ---- gemm.hip
// Plain product stored in the operand dtype (or fp32 when c_f32).  streaming:
// bf16 output written with non-temporal stores, for products that nothing
// reads before they would have left the caches anyway (the weight gradients).
hipError_t launch_gemm_store(int dtype, const GemmDesc& g, void* c, int64_t ldc, bool c_f32,
                             hipStream_t s, bool streaming = false);
// Input projection of the block: columns < qkv_cols (3A for the fused
// projection, 0 for FC1 alone) go to qkv [T, qkv_cols] (and, for the q and
// k columns, their bf16 rounding residual to qk_lo [T, 2A] when qk_lo is not
// null); the FC1 columns go to f [T, F] (pre-activation) and GeLU(f) to
// cat[:, A:].
hipError_t launch_gemm_in_fwd(int dtype, const GemmDesc& g, void* qkv, void* qk_lo, void* f,
                              void* cat, int attn_width, int ffn, int qkv_cols, hipStream_t s);
// Output projection plus optional residual: y = acc (+ x).
hipError_t launch_gemm_out_fwd(int dtype, const GemmDesc& g, const void* x, int add_residual,
                               void* y, hipStream_t s);
// Backward of the output projection w.r.t. cat (dcat = dy w_out^T): columns < A go to dO [T, A];
// FC2 column c is multiplied by GeLU'(f[:, c]) and goes to dz[t * dz_ld + dz_off + c].
hipError_t launch_gemm_dcat(int dtype, const GemmDesc& g, const void* f, void* d_o, void* dz,
                            int attn_width, int ffn, int64_t dz_ld, int64_t dz_off, hipStream_t s);

// ---- swa.hip
struct SwaDesc {
  int batch, seq, n_heads, head_dim, window;
  const void* qkv;   // [T, ld_qkv]: q at col h*d, k at A + h*d, v at 2A + h*d
  int64_t ld_qkv;
  // bf16 only, may be null: [T, 2A] residuals q - bf16(q) | k - bf16(k);
  // the scores then use q_hi k_hi + q_hi k_lo + q_lo k_hi.
  const void* qk_lo = nullptr;
};
hipError_t launch_swa_fwd(int dtype, const SwaDesc& a, void* o, int64_t ldo, float* lse,
                          hipStream_t s);
// dqkv: [T, ld_dqkv] with dq at col h*d, dk at A + h*d, dv at 2A + h*d.
// dvec: fp32 [batch, H, seq] temporary holding rowsum(dO * O).
hipError_t launch_swa_bwd(int dtype, const SwaDesc& a, const void* o, int64_t ldo,
                          const void* d_o, int64_t ld_do, const float* lse, float* dvec,
                          void* dqkv, int64_t ld_dqkv, hipStream_t s);

// ---- lamb.hip
constexpr int kLambMaxTensors = 16;
struct LambBatch {
  float* w[kLambMaxTensors];
  const void* g[kLambMaxTensors];
  float* m[kLambMaxTensors];
  float* v[kLambMaxTensors];
  void* wc[kLambMaxTensors];  // optional bf16 copy of the updated w
  int64_t n[kLambMaxTensors];
  float wd[kLambMaxTensors];
  int gdt[kLambMaxTensors];   // gradient dtype (0 fp32, 1 bf16)
  int blk_start[kLambMaxTensors + 1];  // first block of each tensor; last = total
  int ntensors;
};
struct LambHyper {
  float lr, beta1, beta2, eps, bc1, bc2;  // bc = 1 - beta^step
};
int64_t lamb_blocks_for(int64_t n);
hipError_t launch_lamb(const LambBatch& b, const LambHyper& hp, float* partials, float* ratios,
                       float* ratios_out, hipStream_t s);
hipError_t launch_lamb_norms(const LambBatch& b, const LambHyper& hp, float* partials,
                             double* norms, hipStream_t s);
hipError_t launch_lamb_apply(const LambBatch& b, const LambHyper& hp, const double* norms,
                             float* ratios, float* ratios_out, hipStream_t s);

}  // namespace ptb
