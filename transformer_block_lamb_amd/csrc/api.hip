// C ABI of the library: argument validation, buffer carving and the launch
// sequence of the block's forward and backward and of the LAMB step.
// Declarations and argument documentation: include/ptb.h and
// include/ptb_ops.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/ptb.h"
#include "../../include/ptb_ops.h"
#include "kernels.h"

using namespace ptb;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxMatrixBytes = (int64_t)1 << 31;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t esize(int dtype) { return dtype == PTB_BF16 ? 2 : 4; }

int check_dims(const ptb_dims* d) {
  if (d == nullptr) return PTB_ERR_INVALID_ARG;
  if (d->batch < 1 || d->seq < 1 || d->hidden < 1 || d->n_heads < 1 || d->head_dim < 1 ||
      d->ffn < 1 || d->window < 1)
    return PTB_ERR_INVALID_ARG;
  if (d->dtype != PTB_F32 && d->dtype != PTB_BF16) return PTB_ERR_INVALID_ARG;
  if (!(d->ln_eps >= 0.0f) || !isfinite(d->ln_eps)) return PTB_ERR_INVALID_ARG;
  if (d->add_residual != 0 && d->add_residual != 1) return PTB_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 96 && d->head_dim != 128) return PTB_ERR_UNSUPPORTED;
  if (d->hidden % 8 != 0 || d->ffn % 8 != 0 || d->hidden > 32768) return PTB_ERR_UNSUPPORTED;
  const int64_t T = (int64_t)d->batch * d->seq;
  const int64_t A = (int64_t)d->n_heads * d->head_dim;
  const int64_t N1 = 3 * A + d->ffn, K2 = A + d->ffn;
  const int64_t e = (int64_t)esize(d->dtype);
  if (T > INT32_MAX / 4 || N1 > INT32_MAX / 4) return PTB_ERR_UNSUPPORTED;
  // every matrix addressed by a buffer resource must stay below 2 GiB
  const int64_t widest = N1 > d->hidden ? N1 : d->hidden;
  if (T * widest * 4 >= kMaxMatrixBytes || N1 * d->hidden * e >= kMaxMatrixBytes ||
      K2 * d->hidden * e >= kMaxMatrixBytes)
    return PTB_ERR_UNSUPPORTED;
  return PTB_OK;
}

struct Dims {
  int64_t T, h, A, F, N1, K2, H, D, S, B;
  size_t e;
  explicit Dims(const ptb_dims* d)
      : T((int64_t)d->batch * d->seq), h(d->hidden), A((int64_t)d->n_heads * d->head_dim),
        F(d->ffn), N1(3 * A + F), K2(A + F), H(d->n_heads), D(d->head_dim), S(d->seq),
        B(d->batch), e(esize(d->dtype)) {}
};

// Saved-activation buffer written by forward, read by backward.
// For bf16 it also keeps the bf16 rounding residuals of xn and of q, k, so
// the attention scores are formed at fp32-level accuracy (see the input
// GEMM and the attention kernels).
struct SavedLayout {
  size_t xn, xn_lo, qk_lo, qkv, f, cat, mean, rstd, lse, total;
  explicit SavedLayout(const Dims& d) {
    const bool split = d.e == 2;
    size_t o = 0;
    xn = o;   o += up(d.T * d.h * d.e);
    xn_lo = o; o += split ? up(d.T * d.h * 2) : 0;
    qk_lo = o; o += split ? up(d.T * 2 * d.A * 2) : 0;
    qkv = o;  o += up(d.T * 3 * d.A * d.e);
    f = o;    o += up(d.T * d.F * d.e);
    cat = o;  o += up(d.T * d.K2 * d.e);
    mean = o; o += up(d.T * 4);
    rstd = o; o += up(d.T * 4);
    lse = o;  o += up(d.B * d.H * d.S * 4);
    total = o;
  }
};

// Temporaries of one call: the backward's intermediate gradients, and the
// split-K workspace of the GEMMs, which the forward uses too.  Nothing in it
// outlives a call.
struct ScratchLayout {
  size_t d_o, dz, dxn, dvec, gpart, bpart, gemm_ws, total;
  explicit ScratchLayout(const Dims& d) {
    const int64_t nblk = (d.T + ln_bwd_rows_per_block() - 1) / ln_bwd_rows_per_block();
    size_t o = 0;
    d_o = o;   o += up(d.T * d.A * d.e);
    dz = o;    o += up(d.T * d.N1 * d.e);
    dxn = o;   o += up(d.T * d.h * d.e);
    dvec = o;  o += up(d.B * d.H * d.S * 4);
    gpart = o; o += up(nblk * d.h * 4);
    bpart = o; o += up(nblk * d.h * 4);
    gemm_ws = o; o += d.e == 2 ? kGemmWsBytes : 0;
    total = o;
  }
};

// The attention descriptor of a call.  A window of at least the sequence
// length is plain causal attention, so it is clamped to the sequence length
// here once: the kernels' band arithmetic (query index + window - 1) then
// stays far from the int32 range whatever window the caller passes.
SwaDesc swa_desc(const ptb_dims* dims, const void* qkv, int64_t ld_qkv, const void* qk_lo) {
  const int w = dims->window < dims->seq ? dims->window : dims->seq;
  return SwaDesc{dims->batch, dims->seq, dims->n_heads, dims->head_dim, w, qkv, ld_qkv, qk_lo};
}

// The forward's scratch is optional: null with 0 bytes runs every GEMM on
// whole-tile schedules; otherwise it must be the full, aligned buffer.
int check_fwd_scratch(const void* scratch, size_t bytes, size_t need) {
  if (scratch == nullptr) return bytes == 0 ? PTB_OK : PTB_ERR_INVALID_ARG;
  if (!aligned16(scratch)) return PTB_ERR_INVALID_ARG;
  return bytes >= need ? PTB_OK : PTB_ERR_WORKSPACE;
}

template <typename T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }
template <typename T>
const T* at(const void* base, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? PTB_OK : PTB_ERR_HIP; }

bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr || !aligned16(p)) return false;
  return true;
}

}  // namespace

extern "C" {

const char* ptb_status_string(int s) {
  switch (s) {
    case PTB_OK: return "ok";
    case PTB_ERR_INVALID_ARG: return "invalid argument (null/unaligned pointer or bad size)";
    case PTB_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PTB_ERR_WORKSPACE: return "workspace buffer too small";
    case PTB_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

size_t ptb_saved_bytes(const ptb_dims* d) {
  if (check_dims(d) != PTB_OK) return 0;
  return SavedLayout(Dims(d)).total;
}

size_t ptb_scratch_bytes(const ptb_dims* d) {
  if (check_dims(d) != PTB_OK) return 0;
  return ScratchLayout(Dims(d)).total;
}

int ptb_forward_stage(const ptb_dims* dims, int32_t stage, const void* x, const float* ln_gamma,
                      const float* ln_beta, const void* w_in, const void* w_out, void* y,
                      void* saved, size_t saved_bytes, void* scratch, size_t scratch_bytes,
                      hipStream_t stream) {
  int st = check_dims(dims);
  if (st != PTB_OK) return st;
  if (stage < -1 || stage >= PTB_FWD_STAGES) return PTB_ERR_INVALID_ARG;
  if (!all_aligned({x, ln_gamma, ln_beta, w_in, w_out, y, saved})) return PTB_ERR_INVALID_ARG;
  const Dims d(dims);
  const SavedLayout L(d);
  const ScratchLayout R(d);
  if (saved_bytes < L.total) return PTB_ERR_WORKSPACE;
  st = check_fwd_scratch(scratch, scratch_bytes, R.total);
  if (st != PTB_OK) return st;
  const int dt = dims->dtype;
  void* xn = at<char>(saved, L.xn);
  void* xn_lo = dt == PTB_BF16 ? at<char>(saved, L.xn_lo) : nullptr;
  void* qk_lo = dt == PTB_BF16 ? at<char>(saved, L.qk_lo) : nullptr;
  void* qkv = at<char>(saved, L.qkv);
  void* f = at<char>(saved, L.f);
  void* cat = at<char>(saved, L.cat);
  float* mean = at<float>(saved, L.mean);
  float* rstd = at<float>(saved, L.rstd);
  float* lse = at<float>(saved, L.lse);
  void* ws = dt == PTB_BF16 && scratch != nullptr ? at<char>(scratch, R.gemm_ws) : nullptr;
  const size_t ws_bytes = ws != nullptr ? kGemmWsBytes : 0;
  const SwaDesc sw = swa_desc(dims, qkv, 3 * d.A, qk_lo);
  for (int s = (stage < 0 ? 0 : stage); s < (stage < 0 ? PTB_FWD_STAGES : stage + 1); ++s) {
    hipError_t e = hipSuccess;
    switch (s) {
      case PTB_FWD_LAYERNORM:
        e = launch_ln_fwd(dt, x, ln_gamma, ln_beta, dims->ln_eps, (int)d.T, (int)d.h, xn, xn_lo,
                          mean, rstd, stream);
        break;
      case PTB_FWD_GEMM_IN: {  // [q|k|v|f] = xn w_in^T; GeLU(f) into cat
        // the q and k column tiles take a second pass over xn_lo (bf16 only)
        GemmDesc g{(int)d.T, (int)d.N1, (int)d.h, kKContig, kKContig, xn, d.h, w_in, d.h};
        g.a2 = xn_lo;
        g.n_split = (int)(2 * d.A);
        g.ws = ws;
        g.ws_bytes = ws_bytes;
        e = launch_gemm_in_fwd(dt, g, qkv, qk_lo, f, cat, (int)d.A, (int)d.F, (int)(3 * d.A),
                               stream);
        break;
      }
      case PTB_FWD_ATTENTION:
        e = launch_swa_fwd(dt, sw, cat, d.K2, lse, stream);
        break;
      case PTB_FWD_GEMM_OUT: {  // y = [x] + cat w_out
        GemmDesc g{(int)d.T, (int)d.h, (int)d.K2, kKContig, kMNContig, cat, d.K2, w_out, d.h};
        g.ws = ws;
        g.ws_bytes = ws_bytes;
        e = launch_gemm_out_fwd(dt, g, x, dims->add_residual, y, stream);
        break;
      }
    }
    if (e != hipSuccess) return PTB_ERR_HIP;
  }
  return PTB_OK;
}

int ptb_forward(const ptb_dims* dims, const void* x, const float* ln_gamma, const float* ln_beta,
                const void* w_in, const void* w_out, void* y, void* saved, size_t saved_bytes,
                void* scratch, size_t scratch_bytes, hipStream_t stream) {
  return ptb_forward_stage(dims, -1, x, ln_gamma, ln_beta, w_in, w_out, y, saved, saved_bytes,
                           scratch, scratch_bytes, stream);
}

int ptb_backward_stage(const ptb_dims* dims, int32_t stage, const void* x, const float* ln_gamma,
                       const void* w_in, const void* w_out, const void* saved, size_t saved_bytes,
                       const void* dy, void* dx, float* d_ln_gamma, float* d_ln_beta, void* dw_in,
                       void* dw_out, void* scratch, size_t scratch_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st != PTB_OK) return st;
  if (stage < -1 || stage >= PTB_BWD_STAGES) return PTB_ERR_INVALID_ARG;
  if (!all_aligned({x, ln_gamma, w_in, w_out, saved, dy, dx, d_ln_gamma, d_ln_beta, dw_in,
                    dw_out, scratch}))
    return PTB_ERR_INVALID_ARG;
  const Dims d(dims);
  const SavedLayout L(d);
  const ScratchLayout R(d);
  if (saved_bytes < L.total || scratch_bytes < R.total) return PTB_ERR_WORKSPACE;
  const int dt = dims->dtype;
  const void* xn = at<char>(saved, L.xn);
  const void* qk_lo = dt == PTB_BF16 ? at<char>(saved, L.qk_lo) : nullptr;
  const void* qkv = at<char>(saved, L.qkv);
  const void* f = at<char>(saved, L.f);
  const void* cat = at<char>(saved, L.cat);
  const float* mean = at<float>(saved, L.mean);
  const float* rstd = at<float>(saved, L.rstd);
  const float* lse = at<float>(saved, L.lse);
  void* d_o = at<char>(scratch, R.d_o);
  void* dz = at<char>(scratch, R.dz);
  void* dxn = at<char>(scratch, R.dxn);
  float* dvec = at<float>(scratch, R.dvec);
  float* gpart = at<float>(scratch, R.gpart);
  float* bpart = at<float>(scratch, R.bpart);
  void* ws = dt == PTB_BF16 ? at<char>(scratch, R.gemm_ws) : nullptr;
  const size_t ws_bytes = dt == PTB_BF16 ? kGemmWsBytes : 0;
  const SwaDesc sw = swa_desc(dims, qkv, 3 * d.A, qk_lo);
  for (int s = (stage < 0 ? 0 : stage); s < (stage < 0 ? PTB_BWD_STAGES : stage + 1); ++s) {
    hipError_t e = hipSuccess;
    switch (s) {
      case PTB_BWD_GEMM_DCAT: {  // dcat = dy w_out^T -> dO | dz[:, 3A:] = dg * GeLU'(f)
        GemmDesc g{(int)d.T, (int)d.K2, (int)d.h, kKContig, kKContig, dy, d.h, w_out, d.h};
        g.ws = ws;
        g.ws_bytes = ws_bytes;
        e = launch_gemm_dcat(dt, g, f, d_o, dz, (int)d.A, (int)d.F, d.N1, 3 * d.A, stream);
        break;
      }
      case PTB_BWD_GEMM_DW_OUT: {  // dw_out = cat^T dy
        GemmDesc g{(int)d.K2, (int)d.h, (int)d.T, kMNContig, kMNContig, cat, d.K2, dy, d.h};
        g.ws = ws;
        g.ws_bytes = ws_bytes;
        e = launch_gemm_store(dt, g, dw_out, d.h, false, stream, true);
        break;
      }
      case PTB_BWD_ATTENTION:  // -> dz[:, :3A]
        e = launch_swa_bwd(dt, sw, cat, d.K2, d_o, d.A, lse, dvec, dz, d.N1, stream);
        break;
      case PTB_BWD_GEMM_DW_IN: {  // dw_in = dz^T xn
        GemmDesc g{(int)d.N1, (int)d.h, (int)d.T, kMNContig, kMNContig, dz, d.N1, xn, d.h};
        g.ws = ws;
        g.ws_bytes = ws_bytes;
        e = launch_gemm_store(dt, g, dw_in, d.h, false, stream, true);
        break;
      }
      case PTB_BWD_GEMM_DXN: {  // dxn = dz w_in
        GemmDesc g{(int)d.T, (int)d.h, (int)d.N1, kKContig, kMNContig, dz, d.N1, w_in, d.h};
        g.ws = ws;
        g.ws_bytes = ws_bytes;
        e = launch_gemm_store(dt, g, dxn, d.h, false, stream);
        break;
      }
      case PTB_BWD_LAYERNORM: {  // dx (+ dy), then the deterministic dgamma/dbeta reduce
        e = launch_ln_bwd(dt, x, ln_gamma, mean, rstd, dxn, dims->add_residual ? dy : nullptr, dx,
                          gpart, bpart, (int)d.T, (int)d.h, stream);
        if (e == hipSuccess) {
          const int nblk = (int)((d.T + ln_bwd_rows_per_block() - 1) / ln_bwd_rows_per_block());
          e = launch_ln_bwd_reduce(gpart, bpart, nblk, (int)d.h, d_ln_gamma, d_ln_beta, stream);
        }
        break;
      }
    }
    if (e != hipSuccess) return PTB_ERR_HIP;
  }
  return PTB_OK;
}

int ptb_backward(const ptb_dims* dims, const void* x, const float* ln_gamma, const void* w_in,
                 const void* w_out, const void* saved, size_t saved_bytes, const void* dy,
                 void* dx, float* d_ln_gamma, float* d_ln_beta, void* dw_in, void* dw_out,
                 void* scratch, size_t scratch_bytes, hipStream_t stream) {
  return ptb_backward_stage(dims, -1, x, ln_gamma, w_in, w_out, saved, saved_bytes, dy, dx,
                            d_ln_gamma, d_ln_beta, dw_in, dw_out, scratch, scratch_bytes, stream);
}

// ------------------------------------------------------------------ serial block
// h = x + Attention(LN1(x)); y = h + MLP(LN2(h)) on the same kernels and the
// same w_in / w_out layout as the PTB, with unfused projections.
namespace {

struct SerialSavedLayout {
  size_t xn1, xn1_lo, qk_lo, qkv, cat, hid, xn2, f, mean1, rstd1, mean2, rstd2, lse, total;
  explicit SerialSavedLayout(const Dims& d) {
    const bool split = d.e == 2;
    size_t o = 0;
    xn1 = o;    o += up(d.T * d.h * d.e);
    xn1_lo = o; o += split ? up(d.T * d.h * 2) : 0;
    qk_lo = o;  o += split ? up(d.T * 2 * d.A * 2) : 0;
    qkv = o;    o += up(d.T * 3 * d.A * d.e);
    cat = o;    o += up(d.T * d.K2 * d.e);
    hid = o;    o += up(d.T * d.h * d.e);
    xn2 = o;    o += up(d.T * d.h * d.e);
    f = o;      o += up(d.T * d.F * d.e);
    mean1 = o;  o += up(d.T * 4);
    rstd1 = o;  o += up(d.T * 4);
    mean2 = o;  o += up(d.T * 4);
    rstd2 = o;  o += up(d.T * 4);
    lse = o;    o += up(d.B * d.H * d.S * 4);
    total = o;
  }
};

struct SerialScratchLayout {
  size_t d_o, dz, dxn, dh, dvec, gpart, bpart, gemm_ws, total;
  explicit SerialScratchLayout(const Dims& d) {
    const int64_t nblk = (d.T + ln_bwd_rows_per_block() - 1) / ln_bwd_rows_per_block();
    size_t o = 0;
    d_o = o;   o += up(d.T * d.A * d.e);
    dz = o;    o += up(d.T * d.N1 * d.e);
    dxn = o;   o += up(d.T * d.h * d.e);
    dh = o;    o += up(d.T * d.h * d.e);
    dvec = o;  o += up(d.B * d.H * d.S * 4);
    gpart = o; o += up(nblk * d.h * 4);
    bpart = o; o += up(nblk * d.h * 4);
    gemm_ws = o; o += d.e == 2 ? kGemmWsBytes : 0;
    total = o;
  }
};

int check_serial_dims(const ptb_dims* d) {
  const int st = check_dims(d);
  if (st != PTB_OK) return st;
  // LN2 normalises the whole h, so the serial block has both residuals
  return d->add_residual == 1 ? PTB_OK : PTB_ERR_INVALID_ARG;
}

const char* off(const void* p, int64_t elems, size_t e) {
  return static_cast<const char*>(p) + elems * (int64_t)e;
}

}  // namespace

size_t ptb_serial_saved_bytes(const ptb_dims* d) {
  if (check_serial_dims(d) != PTB_OK) return 0;
  return SerialSavedLayout(Dims(d)).total;
}

size_t ptb_serial_scratch_bytes(const ptb_dims* d) {
  if (check_serial_dims(d) != PTB_OK) return 0;
  return SerialScratchLayout(Dims(d)).total;
}

int ptb_serial_forward(const ptb_dims* dims, const void* x, const float* ln1_gamma,
                       const float* ln1_beta, const float* ln2_gamma, const float* ln2_beta,
                       const void* w_in, const void* w_out, void* y, void* saved,
                       size_t saved_bytes, void* scratch, size_t scratch_bytes,
                       hipStream_t stream) {
  int st = check_serial_dims(dims);
  if (st != PTB_OK) return st;
  if (!all_aligned({x, ln1_gamma, ln1_beta, ln2_gamma, ln2_beta, w_in, w_out, y, saved}))
    return PTB_ERR_INVALID_ARG;
  const Dims d(dims);
  const SerialSavedLayout L(d);
  const SerialScratchLayout R(d);
  if (saved_bytes < L.total) return PTB_ERR_WORKSPACE;
  st = check_fwd_scratch(scratch, scratch_bytes, R.total);
  if (st != PTB_OK) return st;
  const int dt = dims->dtype;
  const bool bf = dt == PTB_BF16;
  void* xn1 = at<char>(saved, L.xn1);
  void* xn1_lo = bf ? at<char>(saved, L.xn1_lo) : nullptr;
  void* qk_lo = bf ? at<char>(saved, L.qk_lo) : nullptr;
  void* qkv = at<char>(saved, L.qkv);
  void* cat = at<char>(saved, L.cat);
  void* hid = at<char>(saved, L.hid);
  void* xn2 = at<char>(saved, L.xn2);
  void* f = at<char>(saved, L.f);
  void* ws = bf && scratch != nullptr ? at<char>(scratch, R.gemm_ws) : nullptr;
  const size_t wsb = ws != nullptr ? kGemmWsBytes : 0;
  const SwaDesc sw = swa_desc(dims, qkv, 3 * d.A, qk_lo);
  hipError_t e = launch_ln_fwd(dt, x, ln1_gamma, ln1_beta, dims->ln_eps, (int)d.T, (int)d.h, xn1,
                               xn1_lo, at<float>(saved, L.mean1), at<float>(saved, L.rstd1),
                               stream);
  if (e == hipSuccess) {  // [q|k|v] = xn1 w_qkv^T (q, k with the second pass over xn1_lo)
    GemmDesc g{(int)d.T, (int)(3 * d.A), (int)d.h, kKContig, kKContig, xn1, d.h, w_in, d.h};
    g.a2 = xn1_lo;
    g.n_split = (int)(2 * d.A);
    g.ws = ws;
    g.ws_bytes = wsb;
    e = launch_gemm_in_fwd(dt, g, qkv, qk_lo, f, cat, (int)d.A, (int)d.F, (int)(3 * d.A), stream);
  }
  if (e == hipSuccess) e = launch_swa_fwd(dt, sw, cat, d.K2, at<float>(saved, L.lse), stream);
  if (e == hipSuccess) {  // h = x + O w_o
    GemmDesc g{(int)d.T, (int)d.h, (int)d.A, kKContig, kMNContig, cat, d.K2, w_out, d.h};
    g.ws = ws;
    g.ws_bytes = wsb;
    e = launch_gemm_out_fwd(dt, g, x, 1, hid, stream);
  }
  if (e == hipSuccess)
    e = launch_ln_fwd(dt, hid, ln2_gamma, ln2_beta, dims->ln_eps, (int)d.T, (int)d.h, xn2,
                      nullptr, at<float>(saved, L.mean2), at<float>(saved, L.rstd2), stream);
  if (e == hipSuccess) {  // f = xn2 w_fc1^T, GeLU(f) into cat[:, A:]
    GemmDesc g{(int)d.T, (int)d.F, (int)d.h, kKContig, kKContig, xn2, d.h,
               off(w_in, 3 * d.A * d.h, d.e), d.h};
    g.ws = ws;
    g.ws_bytes = wsb;
    e = launch_gemm_in_fwd(dt, g, qkv, nullptr, f, cat, (int)d.A, (int)d.F, 0, stream);
  }
  if (e == hipSuccess) {  // y = h + GeLU(f) w_fc2
    GemmDesc g{(int)d.T, (int)d.h, (int)d.F, kKContig, kMNContig, off(cat, d.A, d.e), d.K2,
               off(w_out, d.A * d.h, d.e), d.h};
    g.ws = ws;
    g.ws_bytes = wsb;
    e = launch_gemm_out_fwd(dt, g, hid, 1, y, stream);
  }
  return e == hipSuccess ? PTB_OK : PTB_ERR_HIP;
}

int ptb_serial_backward(const ptb_dims* dims, const void* x, const float* ln1_gamma,
                        const float* ln2_gamma, const void* w_in, const void* w_out,
                        const void* saved, size_t saved_bytes, const void* dy, void* dx,
                        float* d_ln1_gamma, float* d_ln1_beta, float* d_ln2_gamma,
                        float* d_ln2_beta, void* dw_in, void* dw_out, void* scratch,
                        size_t scratch_bytes, hipStream_t stream) {
  int st = check_serial_dims(dims);
  if (st != PTB_OK) return st;
  if (!all_aligned({x, ln1_gamma, ln2_gamma, w_in, w_out, saved, dy, dx, d_ln1_gamma, d_ln1_beta,
                    d_ln2_gamma, d_ln2_beta, dw_in, dw_out, scratch}))
    return PTB_ERR_INVALID_ARG;
  const Dims d(dims);
  const SerialSavedLayout L(d);
  const SerialScratchLayout R(d);
  if (saved_bytes < L.total || scratch_bytes < R.total) return PTB_ERR_WORKSPACE;
  const int dt = dims->dtype;
  const bool bf = dt == PTB_BF16;
  const void* xn1 = at<char>(saved, L.xn1);
  const void* qk_lo = bf ? at<char>(saved, L.qk_lo) : nullptr;
  const void* qkv = at<char>(saved, L.qkv);
  const void* cat = at<char>(saved, L.cat);
  const void* hid = at<char>(saved, L.hid);
  const void* xn2 = at<char>(saved, L.xn2);
  const void* f = at<char>(saved, L.f);
  void* d_o = at<char>(scratch, R.d_o);
  void* dz = at<char>(scratch, R.dz);
  void* dxn = at<char>(scratch, R.dxn);
  void* dh = at<char>(scratch, R.dh);
  float* gpart = at<float>(scratch, R.gpart);
  float* bpart = at<float>(scratch, R.bpart);
  void* ws = bf ? at<char>(scratch, R.gemm_ws) : nullptr;
  const size_t wsb = bf ? kGemmWsBytes : 0;
  const int nblk = (int)((d.T + ln_bwd_rows_per_block() - 1) / ln_bwd_rows_per_block());
  const SwaDesc sw = swa_desc(dims, qkv, 3 * d.A, qk_lo);
  auto gemm = [&](int M, int N, int K, int al, int bl, const void* a, int64_t lda, const void* b,
                  int64_t ldb) {
    GemmDesc g{M, N, K, al, bl, a, lda, b, ldb};
    g.ws = ws;
    g.ws_bytes = wsb;
    return g;
  };
  char* dw_in_c = static_cast<char*>(dw_in);
  char* dw_out_c = static_cast<char*>(dw_out);
  // MLP sub-layer: dw_fc2 = GeLU(f)^T dy; df = (dy w_fc2^T) GeLU'(f) into dz[:, 3A:]
  hipError_t e = launch_gemm_store(
      dt, gemm((int)d.F, (int)d.h, (int)d.T, kMNContig, kMNContig, off(cat, d.A, d.e), d.K2, dy, d.h),
      dw_out_c + d.A * d.h * d.e, d.h, false, stream, true);
  if (e == hipSuccess)
    e = launch_gemm_dcat(dt, gemm((int)d.T, (int)d.F, (int)d.h, kKContig, kKContig, dy, d.h,
                                  off(w_out, d.A * d.h, d.e), d.h),
                         f, d_o, dz, 0, (int)d.F, d.N1, 3 * d.A, stream);
  if (e == hipSuccess)  // dw_fc1 = df^T xn2
    e = launch_gemm_store(dt, gemm((int)d.F, (int)d.h, (int)d.T, kMNContig, kMNContig,
                                   off(dz, 3 * d.A, d.e), d.N1, xn2, d.h),
                          dw_in_c + 3 * d.A * d.h * d.e, d.h, false, stream, true);
  if (e == hipSuccess)  // dxn2 = df w_fc1
    e = launch_gemm_store(dt, gemm((int)d.T, (int)d.h, (int)d.F, kKContig, kMNContig,
                                   off(dz, 3 * d.A, d.e), d.N1, off(w_in, 3 * d.A * d.h, d.e), d.h),
                          dxn, d.h, false, stream);
  if (e == hipSuccess)  // dh = dy + LN2 backward
    e = launch_ln_bwd(dt, hid, ln2_gamma, at<float>(saved, L.mean2), at<float>(saved, L.rstd2),
                      dxn, dy, dh, gpart, bpart, (int)d.T, (int)d.h, stream);
  if (e == hipSuccess)
    e = launch_ln_bwd_reduce(gpart, bpart, nblk, (int)d.h, d_ln2_gamma, d_ln2_beta, stream);
  // attention sub-layer: dw_o = O^T dh; dO = dh w_o^T
  if (e == hipSuccess)
    e = launch_gemm_store(dt, gemm((int)d.A, (int)d.h, (int)d.T, kMNContig, kMNContig, cat, d.K2,
                                   dh, d.h),
                          dw_out, d.h, false, stream, true);
  if (e == hipSuccess)
    e = launch_gemm_dcat(dt, gemm((int)d.T, (int)d.A, (int)d.h, kKContig, kKContig, dh, d.h, w_out,
                                  d.h),
                         f, d_o, dz, (int)d.A, (int)d.F, d.N1, 3 * d.A, stream);
  if (e == hipSuccess)  // -> dz[:, :3A]
    e = launch_swa_bwd(dt, sw, cat, d.K2, d_o, d.A, at<float>(saved, L.lse),
                       at<float>(scratch, R.dvec), dz, d.N1, stream);
  if (e == hipSuccess)  // dw_qkv = dqkv^T xn1
    e = launch_gemm_store(dt, gemm((int)(3 * d.A), (int)d.h, (int)d.T, kMNContig, kMNContig, dz,
                                   d.N1, xn1, d.h),
                          dw_in, d.h, false, stream, true);
  if (e == hipSuccess)  // dxn1 = dqkv w_qkv
    e = launch_gemm_store(dt, gemm((int)d.T, (int)d.h, (int)(3 * d.A), kKContig, kMNContig, dz,
                                   d.N1, w_in, d.h),
                          dxn, d.h, false, stream);
  if (e == hipSuccess)  // dx = dh + LN1 backward
    e = launch_ln_bwd(dt, x, ln1_gamma, at<float>(saved, L.mean1), at<float>(saved, L.rstd1), dxn,
                      dh, dx, gpart, bpart, (int)d.T, (int)d.h, stream);
  if (e == hipSuccess)
    e = launch_ln_bwd_reduce(gpart, bpart, nblk, (int)d.h, d_ln1_gamma, d_ln1_beta, stream);
  return e == hipSuccess ? PTB_OK : PTB_ERR_HIP;
}

size_t lamb_scratch_bytes(const lamb_tensor* t, int32_t n) {
  if (t == nullptr || n < 1) return 0;
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    if (t[i].n < 0) return 0;
    blocks += lamb_blocks_for(t[i].n);
  }
  return up((size_t)blocks * 2 * sizeof(float)) + up((size_t)n * sizeof(float));
}

}  // extern "C"

namespace {

// Checks a LAMB call (the gradient may be absent only when `need_grad` is
// false) and fills the hyper-parameters and the total block count.
int lamb_check(const lamb_tensor* t, int32_t n, float lr, float beta1, float beta2, float eps,
               int64_t step, void* scratch, size_t scratch_bytes, bool need_grad, LambHyper& hp,
               int64_t& total_blocks) {
  if (t == nullptr || n < 1 || step < 1) return PTB_ERR_INVALID_ARG;
  // eps > 0: with eps = 0 a zero gradient on fresh moments makes u = 0 / 0
  if (!(beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f && eps > 0.f &&
        isfinite(eps) && isfinite(lr)))
    return PTB_ERR_INVALID_ARG;
  if (scratch == nullptr || !aligned16(scratch)) return PTB_ERR_INVALID_ARG;
  total_blocks = 0;
  for (int i = 0; i < n; ++i) {
    if (t[i].n < 1 || !all_aligned({t[i].w, t[i].m, t[i].v})) return PTB_ERR_INVALID_ARG;
    if ((need_grad || t[i].g != nullptr) && !all_aligned({t[i].g})) return PTB_ERR_INVALID_ARG;
    if (t[i].w_bf16 != nullptr && !aligned16(t[i].w_bf16)) return PTB_ERR_INVALID_ARG;
    if (t[i].grad_dtype != PTB_F32 && t[i].grad_dtype != PTB_BF16) return PTB_ERR_INVALID_ARG;
    if (!isfinite(t[i].weight_decay)) return PTB_ERR_INVALID_ARG;
    total_blocks += lamb_blocks_for(t[i].n);
  }
  if (total_blocks > INT32_MAX / 2) return PTB_ERR_UNSUPPORTED;
  if (scratch_bytes < lamb_scratch_bytes(t, n)) return PTB_ERR_WORKSPACE;
  hp.lr = lr; hp.beta1 = beta1; hp.beta2 = beta2; hp.eps = eps;
  hp.bc1 = (float)(1.0 - pow((double)beta1, (double)step));
  hp.bc2 = (float)(1.0 - pow((double)beta2, (double)step));
  if (!(hp.bc1 > 0.f && hp.bc2 > 0.f)) return PTB_ERR_INVALID_ARG;
  return PTB_OK;
}

// Runs `launch(batch, first tensor, first block)` over the tensors in
// groups of at most kLambMaxTensors (one kernel-argument table each).
template <class F>
int lamb_batches(const lamb_tensor* t, int32_t n, F&& launch) {
  int64_t blk_off = 0;
  for (int first = 0; first < n; first += kLambMaxTensors) {
    LambBatch b;
    memset(&b, 0, sizeof(b));
    b.ntensors = n - first < kLambMaxTensors ? n - first : kLambMaxTensors;
    int blk = 0;
    for (int i = 0; i < b.ntensors; ++i) {
      const lamb_tensor& ti = t[first + i];
      b.w[i] = ti.w; b.g[i] = ti.g; b.m[i] = ti.m; b.v[i] = ti.v; b.wc[i] = ti.w_bf16;
      b.n[i] = ti.n; b.wd[i] = ti.weight_decay; b.gdt[i] = ti.grad_dtype;
      b.blk_start[i] = blk;
      blk += (int)lamb_blocks_for(ti.n);
    }
    b.blk_start[b.ntensors] = blk;
    if (launch(b, first, blk_off) != hipSuccess) return PTB_ERR_HIP;
    blk_off += blk;
  }
  return PTB_OK;
}

}  // namespace

extern "C" {

int lamb_step(const lamb_tensor* t, int32_t n, float lr, float beta1, float beta2, float eps,
              int64_t step, float* ratios_out, void* scratch, size_t scratch_bytes,
              hipStream_t stream) {
  LambHyper hp;
  int64_t total_blocks;
  const int st =
      lamb_check(t, n, lr, beta1, beta2, eps, step, scratch, scratch_bytes, true, hp, total_blocks);
  if (st != PTB_OK) return st;
  if (ratios_out != nullptr && (reinterpret_cast<uintptr_t>(ratios_out) & 3u))
    return PTB_ERR_INVALID_ARG;
  float* partials = static_cast<float*>(scratch);
  float* ratios = at<float>(scratch, up((size_t)total_blocks * 2 * sizeof(float)));
  return lamb_batches(t, n, [&](const LambBatch& b, int first, int64_t blk_off) {
    return launch_lamb(b, hp, partials + 2 * blk_off, ratios + first,
                       ratios_out ? ratios_out + first : nullptr, stream);
  });
}

int lamb_shard_norms(const lamb_tensor* t, int32_t n, float beta1, float beta2, float eps,
                     int64_t step, double* norms_out, void* scratch, size_t scratch_bytes,
                     hipStream_t stream) {
  LambHyper hp;
  int64_t total_blocks;
  const int st = lamb_check(t, n, 0.f, beta1, beta2, eps, step, scratch, scratch_bytes, true, hp,
                            total_blocks);
  if (st != PTB_OK) return st;
  if (norms_out == nullptr || (reinterpret_cast<uintptr_t>(norms_out) & 7u))
    return PTB_ERR_INVALID_ARG;
  float* partials = static_cast<float*>(scratch);
  return lamb_batches(t, n, [&](const LambBatch& b, int first, int64_t blk_off) {
    return launch_lamb_norms(b, hp, partials + 2 * blk_off, norms_out + 2 * first, stream);
  });
}

int lamb_shard_apply(const lamb_tensor* t, int32_t n, float lr, float beta1, float beta2,
                     float eps, int64_t step, const double* norms, float* ratios_out,
                     void* scratch, size_t scratch_bytes, hipStream_t stream) {
  LambHyper hp;
  int64_t total_blocks;
  const int st = lamb_check(t, n, lr, beta1, beta2, eps, step, scratch, scratch_bytes, false, hp,
                            total_blocks);
  if (st != PTB_OK) return st;
  if (norms == nullptr || (reinterpret_cast<uintptr_t>(norms) & 7u)) return PTB_ERR_INVALID_ARG;
  if (ratios_out != nullptr && (reinterpret_cast<uintptr_t>(ratios_out) & 3u))
    return PTB_ERR_INVALID_ARG;
  float* ratios = at<float>(scratch, up((size_t)total_blocks * 2 * sizeof(float)));
  return lamb_batches(t, n, [&](const LambBatch& b, int first, int64_t) {
    return launch_lamb_apply(b, hp, norms + 2 * first, ratios + first,
                             ratios_out ? ratios_out + first : nullptr, stream);
  });
}

// ------------------------------------------------------------------ components
int ptb_layernorm_forward(int32_t dtype, int32_t rows, int32_t width, const void* x,
                          const float* gamma, const float* beta, float eps, void* xn,
                          float* mean, float* rstd, hipStream_t stream) {
  if ((dtype != PTB_F32 && dtype != PTB_BF16) || rows < 1 || width < 8 || width % 8 != 0 ||
      width > 32768 || !(eps >= 0.f))
    return PTB_ERR_INVALID_ARG;
  if (!all_aligned({x, gamma, beta, xn, mean, rstd})) return PTB_ERR_INVALID_ARG;
  return hip_status(
      launch_ln_fwd(dtype, x, gamma, beta, eps, rows, width, xn, nullptr, mean, rstd, stream));
}

size_t ptb_layernorm_scratch_bytes(int32_t rows, int32_t width) {
  if (rows < 1 || width < 8 || width % 8 != 0 || width > 32768) return 0;
  const int64_t nblk = ((int64_t)rows + ln_bwd_rows_per_block() - 1) / ln_bwd_rows_per_block();
  return 2 * up((size_t)nblk * width * 4);
}

int ptb_layernorm_backward(int32_t dtype, int32_t rows, int32_t width, const void* x,
                           const float* gamma, const float* mean, const float* rstd,
                           const void* dxn, const void* dy, void* dx, float* dgamma,
                           float* dbeta, void* scratch, size_t scratch_bytes,
                           hipStream_t stream) {
  if (dtype != PTB_F32 && dtype != PTB_BF16) return PTB_ERR_INVALID_ARG;
  const size_t need = ptb_layernorm_scratch_bytes(rows, width);
  if (need == 0) return PTB_ERR_INVALID_ARG;
  if ((int64_t)rows * width * 4 >= kMaxMatrixBytes) return PTB_ERR_UNSUPPORTED;
  if (!all_aligned({x, gamma, mean, rstd, dxn, dx, dgamma, dbeta, scratch}))
    return PTB_ERR_INVALID_ARG;
  if (dy != nullptr && !aligned16(dy)) return PTB_ERR_INVALID_ARG;
  if (scratch_bytes < need) return PTB_ERR_WORKSPACE;
  const int nblk = (rows + ln_bwd_rows_per_block() - 1) / ln_bwd_rows_per_block();
  float* gpart = static_cast<float*>(scratch);
  float* bpart = at<float>(scratch, need / 2);
  hipError_t e = launch_ln_bwd(dtype, x, gamma, mean, rstd, dxn, dy, dx, gpart, bpart, rows,
                               width, stream);
  if (e == hipSuccess) e = launch_ln_bwd_reduce(gpart, bpart, nblk, width, dgamma, dbeta, stream);
  return hip_status(e);
}

size_t ptb_gemm_workspace_bytes(void) { return kGemmWsBytes; }

int ptb_gemm(int32_t dtype, int32_t a_layout, int32_t b_layout, int32_t M, int32_t N, int32_t K,
             const void* a, int64_t lda, const void* b, int64_t ldb, void* c, int64_t ldc,
             int32_t c_f32, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if ((dtype != PTB_F32 && dtype != PTB_BF16) || M < 1 || N < 1 || K < 1) return PTB_ERR_INVALID_ARG;
  if ((a_layout != 0 && a_layout != 1) || (b_layout != 0 && b_layout != 1)) return PTB_ERR_INVALID_ARG;
  if (!all_aligned({a, b, c})) return PTB_ERR_INVALID_ARG;
  if (ldc < N || lda < (a_layout == 0 ? K : M) || ldb < (b_layout == 0 ? K : N))
    return PTB_ERR_INVALID_ARG;
  if (dtype == PTB_BF16) {
    // 16-byte vectors along the contiguous dimension of each operand
    if (lda % 8 || ldb % 8 || ldc % 8) return PTB_ERR_UNSUPPORTED;  // + 16-byte output chunks
    if ((a_layout == 0 ? K : M) % 8 || (b_layout == 0 ? K : N) % 8) return PTB_ERR_UNSUPPORTED;
    const int64_t ea = a_layout == 0 ? (int64_t)M * lda : (int64_t)K * lda;
    const int64_t eb = b_layout == 0 ? (int64_t)N * ldb : (int64_t)K * ldb;
    if (ea * 2 >= kMaxMatrixBytes || eb * 2 >= kMaxMatrixBytes) return PTB_ERR_UNSUPPORTED;
  } else if (c_f32 == 0) {
    c_f32 = 1;  // fp32 operands always produce fp32
  }
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) % 256 != 0 ||
                                workspace_bytes < kGemmWsBytes))
    return PTB_ERR_WORKSPACE;
  GemmDesc g{M, N, K, a_layout, b_layout, a, lda, b, ldb};
  if (dtype == PTB_BF16) {
    g.ws = workspace;
    g.ws_bytes = workspace_bytes;
  }
  return hip_status(launch_gemm_store(dtype, g, c, ldc, c_f32 != 0, stream));
}

int ptb_swa_forward(const ptb_dims* dims, const void* qkv, void* o, int64_t ldo, float* lse,
                    hipStream_t stream) {
  int st = check_dims(dims);
  if (st != PTB_OK) return st;
  if (!all_aligned({qkv, o, lse})) return PTB_ERR_INVALID_ARG;
  const Dims d(dims);
  if (ldo < d.A || ldo % 8) return PTB_ERR_INVALID_ARG;
  const SwaDesc sw = swa_desc(dims, qkv, 3 * d.A, nullptr);
  return hip_status(launch_swa_fwd(dims->dtype, sw, o, ldo, lse, stream));
}

int ptb_swa_backward(const ptb_dims* dims, const void* qkv, const void* o, int64_t ldo,
                     const void* d_o, const float* lse, void* dqkv, float* dvec,
                     hipStream_t stream) {
  int st = check_dims(dims);
  if (st != PTB_OK) return st;
  if (!all_aligned({qkv, o, d_o, lse, dqkv, dvec})) return PTB_ERR_INVALID_ARG;
  const Dims d(dims);
  if (ldo < d.A || ldo % 8) return PTB_ERR_INVALID_ARG;
  const SwaDesc sw = swa_desc(dims, qkv, 3 * d.A, nullptr);
  return hip_status(
      launch_swa_bwd(dims->dtype, sw, o, ldo, d_o, d.A, lse, dvec, dqkv, 3 * d.A, stream));
}

}  // extern "C"
