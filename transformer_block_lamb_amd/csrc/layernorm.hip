// The one shared pre-LayerNorm of the parallel block (MegaScale study guide,
// ch.2 §2.2 technique table, PTB row: the same LN(x) feeds the MLP and the
// attention branch), forward and backward.
//
// Forward: one workgroup of 512 threads per token row; the row stays in
// registers (NV 16-byte vectors per thread), the mean and then the biased
// variance of the centred values are block reductions; xn is written in the
// activation dtype and the row's mean and 1/sqrt(var + eps) in fp32.  For
// bf16, the rounding residual xn - bf16(xn) can be written too (xn_lo).
//
// Backward: one workgroup per ROWS_PER_BLOCK consecutive rows; dxn comes in
// the activation dtype (bf16 for bf16 runs).  For each row
//   xhat = (x - mean) * rstd, dxhat = dxn * gamma,
//   dx = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat)) [+ dy]
// and each thread accumulates its columns' dgamma = sum dxn * xhat and
// dbeta = sum dxn over the block's rows in registers; the per-block partial
// rows are then summed in a fixed order by a second kernel, so the result is
// deterministic.  Both kernels are HBM-bound streaming passes.
#include "common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr int kLnThreads = 512;
constexpr int kLnWaves = kLnThreads / 64;
constexpr int kRowsPerBlock = 8;

// Loads one row's NV 16-byte vectors per thread (zeros past the width).
template <typename T, int NV>
__device__ __forceinline__ void load_row(const T* r, int nvec, float (&v)[NV][8]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + kLnThreads * i;
    if (vi < nvec) {
      Vec8<T>::load(r + vi * 8, v[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    }
  }
}

// Eight values kept as loaded (bf16 stays packed, halving the registers a
// prefetched row needs); get() widens them to fp32.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { u = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void get(float (&o)[8]) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void get(float (&o)[8]) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};
template <typename T, int NV>
__device__ __forceinline__ void load_raw(const T* r, int nvec, Raw8<T> (&v)[NV]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + kLnThreads * i;
    if (vi < nvec) v[i].load(r + vi * 8); else v[i].zero();
  }
}

// ROWS_PER_BLOCK consecutive rows per workgroup; the next row's x, dxn and
// dy are loaded while the current row is reduced (launched while those
// registers fit: up to 3 vectors per thread for bf16 rows, 2 for fp32).
template <typename T, int NV>
__global__ __launch_bounds__(kLnThreads) void ln_bwd_kernel(
    const T* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ mean,
    const float* __restrict__ rstd, const T* __restrict__ dxn, const T* __restrict__ dy,
    T* __restrict__ dx, float* __restrict__ gpart, float* __restrict__ bpart, int rows,
    int width) {
  __shared__ float red[2 * kLnWaves];
  const int nvec = width >> 3;
  const int r0 = blockIdx.x * kRowsPerBlock;
  const int rend = min(rows, r0 + kRowsPerBlock);
  const float inv_w = 1.0f / (float)width;
  float ag[NV][8], ab[NV][8], gm[NV][8];
  load_row<float, NV>(gamma, nvec, gm);
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) { ag[i][e] = 0.f; ab[i][e] = 0.f; }
  Raw8<T> xr[NV], yr[NV], nxr[NV], nyr[NV];
  Raw8<T> dr[NV], ndr[NV];
  if (r0 < rend) {
    load_raw<T, NV>(x + (int64_t)r0 * width, nvec, xr);
    load_raw<T, NV>(dxn + (int64_t)r0 * width, nvec, dr);
    if (dy != nullptr) load_raw<T, NV>(dy + (int64_t)r0 * width, nvec, yr);
  }
  for (int row = r0; row < rend; ++row) {  // uniform over the block
    if (row + 1 < rend) {
      load_raw<T, NV>(x + (int64_t)(row + 1) * width, nvec, nxr);
      load_raw<T, NV>(dxn + (int64_t)(row + 1) * width, nvec, ndr);
      if (dy != nullptr) load_raw<T, NV>(dy + (int64_t)(row + 1) * width, nvec, nyr);
    }
    const float mu = mean[row], rs = rstd[row];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const bool in = threadIdx.x + kLnThreads * i < nvec;
      float xv[8], dv[8];
      xr[i].get(xv);
      dr[i].get(dv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xh = in ? (xv[e] - mu) * rs : 0.f;
        const float dxh = dv[e] * gm[i][e];
        s1 += dxh;
        s2 += dxh * xh;
        ag[i][e] += dv[e] * xh;
        ab[i][e] += dv[e];
      }
    }
    block_sum2<kLnWaves>(s1, s2, red);
    const float m1 = s1 * inv_w, m2 = s2 * inv_w;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = threadIdx.x + kLnThreads * i;
      if (vi < nvec) {
        float xv[8], dv[8], o[8];
        xr[i].get(xv);
        dr[i].get(dv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (xv[e] - mu) * rs;
          o[e] = rs * (dv[e] * gm[i][e] - m1 - xh * m2);
        }
        if (dy != nullptr) {
          float yv[8];
          yr[i].get(yv);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] += yv[e];
        }
        Vec8<T>::store(dx + (int64_t)row * width + vi * 8, o);
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      xr[i] = nxr[i];
      dr[i] = ndr[i];
      yr[i] = nyr[i];
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + kLnThreads * i;
    if (vi < nvec) {
      Vec8<float>::store(gpart + (int64_t)blockIdx.x * width + vi * 8, ag[i]);
      Vec8<float>::store(bpart + (int64_t)blockIdx.x * width + vi * 8, ab[i]);
    }
  }
}

// Forward: each workgroup normalises kFwdRows consecutive rows; the next
// row's loads are issued before the current row is reduced and stored, so
// one row's stores overlap the next row's loads.
constexpr int kFwdRows = 2;
template <typename T, int NV>
__device__ __forceinline__ void ln_fwd_row(const Raw8<T> (&raw)[NV], const float* __restrict__ gamma,
                                           const float* __restrict__ beta, float eps, int width,
                                           int row, T* __restrict__ xn, T* __restrict__ xn_lo,
                                           float* __restrict__ mean_out,
                                           float* __restrict__ rstd_out, float* red);

template <typename T, int NV>
__global__ __launch_bounds__(kLnThreads) void ln_fwd_kernel(const T* __restrict__ x,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ beta,
                                                            float eps, int rows, int width,
                                                            T* __restrict__ xn,
                                                            T* __restrict__ xn_lo,
                                                            float* __restrict__ mean_out,
                                                            float* __restrict__ rstd_out) {
  __shared__ float red[kLnWaves];
  const int nvec = width >> 3;
  const int r0 = blockIdx.x * kFwdRows;
  const int rend = min(rows, r0 + kFwdRows);
  Raw8<T> cur[NV], nxt[NV];
  load_raw<T, NV>(x + (int64_t)r0 * width, nvec, cur);
  for (int row = r0; row < rend; ++row) {  // uniform over the block
    if (row + 1 < rend) load_raw<T, NV>(x + (int64_t)(row + 1) * width, nvec, nxt);
    ln_fwd_row<T, NV>(cur, gamma, beta, eps, width, row, xn, xn_lo, mean_out, rstd_out, red);
#pragma unroll
    for (int i = 0; i < NV; ++i) cur[i] = nxt[i];
  }
}

template <typename T, int NV>
__device__ __forceinline__ void ln_fwd_row(const Raw8<T> (&raw)[NV], const float* __restrict__ gamma,
                                           const float* __restrict__ beta, float eps, int width,
                                           int row, T* __restrict__ xn, T* __restrict__ xn_lo,
                                           float* __restrict__ mean_out,
                                           float* __restrict__ rstd_out, float* red) {
  const int nvec = width >> 3;
  float v[NV][8];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    raw[i].get(v[i]);  // zeros past the width
#pragma unroll
    for (int e = 0; e < 8; ++e) s += v[i][e];
  }
  const float inv_w = 1.0f / (float)width;
  const float mean = block_sum<kLnWaves>(s, red) * inv_w;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + kLnThreads * i;
    if (vi < nvec) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = v[i][e] - mean;
        q += c * c;
      }
    }
  }
  const float var = block_sum<kLnWaves>(q, red) * inv_w;
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + kLnThreads * i;
    if (vi < nvec) {
      float g[8], b[8], o[8];
      Vec8<float>::load(gamma + vi * 8, g);
      Vec8<float>::load(beta + vi * 8, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[i][e] - mean) * rstd * g[e] + b[e];
      Vec8<T>::store(xn + (int64_t)row * width + vi * 8, o);
      if (xn_lo != nullptr) {
        float lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = o[e] - Elt<T>::ld_rounded(o[e]);
        Vec8<T>::store(xn_lo + (int64_t)row * width + vi * 8, lo);
      }
    }
  }
  if (threadIdx.x == 0) {
    mean_out[row] = mean;
    rstd_out[row] = rstd;
  }
}

// Backward for wider rows: the same arithmetic, one row at a time without
// the next-row loads.
template <typename T, int NV>
__global__ __launch_bounds__(kLnThreads) void ln_bwd_plain_kernel(
    const T* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ mean,
    const float* __restrict__ rstd, const T* __restrict__ dxn, const T* __restrict__ dy,
    T* __restrict__ dx, float* __restrict__ gpart, float* __restrict__ bpart, int rows,
    int width) {
  __shared__ float red[2 * kLnWaves];
  const int nvec = width >> 3;
  const int r0 = blockIdx.x * kRowsPerBlock;
  const float inv_w = 1.0f / (float)width;
  float ag[NV][8], ab[NV][8], gm[NV][8];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + kLnThreads * i;
#pragma unroll
    for (int e = 0; e < 8; ++e) { ag[i][e] = 0.f; ab[i][e] = 0.f; gm[i][e] = 0.f; }
    if (vi < nvec) Vec8<float>::load(gamma + vi * 8, gm[i]);
  }
  for (int rr = 0; rr < kRowsPerBlock; ++rr) {
    const int row = r0 + rr;
    if (row >= rows) break;  // uniform over the block
    const float mu = mean[row], rs = rstd[row];
    float xh[NV][8], dxh[NV][8];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = threadIdx.x + kLnThreads * i;
      if (vi < nvec) {
        float xv[8], dv[8];
        Vec8<T>::load(x + (int64_t)row * width + vi * 8, xv);
        Vec8<T>::load(dxn + (int64_t)row * width + vi * 8, dv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xh[i][e] = (xv[e] - mu) * rs;
          dxh[i][e] = dv[e] * gm[i][e];
          s1 += dxh[i][e];
          s2 += dxh[i][e] * xh[i][e];
          ag[i][e] += dv[e] * xh[i][e];
          ab[i][e] += dv[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { xh[i][e] = 0.f; dxh[i][e] = 0.f; }
      }
    }
    block_sum2<kLnWaves>(s1, s2, red);
    const float m1 = s1 * inv_w, m2 = s2 * inv_w;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vi = threadIdx.x + kLnThreads * i;
      if (vi < nvec) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = rs * (dxh[i][e] - m1 - xh[i][e] * m2);
        if (dy != nullptr) {
          float d[8];
          Vec8<T>::load(dy + (int64_t)row * width + vi * 8, d);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] += d[e];
        }
        Vec8<T>::store(dx + (int64_t)row * width + vi * 8, o);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = threadIdx.x + kLnThreads * i;
    if (vi < nvec) {
      Vec8<float>::store(gpart + (int64_t)blockIdx.x * width + vi * 8, ag[i]);
      Vec8<float>::store(bpart + (int64_t)blockIdx.x * width + vi * 8, ab[i]);
    }
  }
}

// Column sums of the per-block partials.  A workgroup owns 64 columns; its
// 16 row groups each add every 16th partial row in order, and the 16 group
// sums are then added in group order, so the result is deterministic.
constexpr int kRedCols = 64, kRedGroups = 16;
__global__ __launch_bounds__(kRedCols * kRedGroups) void ln_bwd_reduce_kernel(
    const float* __restrict__ gpart, const float* __restrict__ bpart, int nblk, int width,
    float* __restrict__ dgamma, float* __restrict__ dbeta) {
  __shared__ float sg_s[kRedGroups][kRedCols], sb_s[kRedGroups][kRedCols];
  const int cl = threadIdx.x % kRedCols, grp = threadIdx.x / kRedCols;
  const int c = blockIdx.x * kRedCols + cl;
  float sg = 0.f, sb = 0.f;
  if (c < width) {
    for (int b = grp; b < nblk; b += kRedGroups) {
      sg += gpart[(int64_t)b * width + c];
      sb += bpart[(int64_t)b * width + c];
    }
  }
  sg_s[grp][cl] = sg;
  sb_s[grp][cl] = sb;
  __syncthreads();
  if (grp == 0 && c < width) {
    float tg = 0.f, tb = 0.f;
#pragma unroll
    for (int g = 0; g < kRedGroups; ++g) {
      tg += sg_s[g][cl];
      tb += sb_s[g][cl];
    }
    dgamma[c] = tg;
    dbeta[c] = tb;
  }
}

template <typename T, int NV>
hipError_t fwd_nv(const void* x, const float* g, const float* b, float eps, int rows, int width,
                  void* xn, void* xn_lo, float* mean, float* rstd, hipStream_t s) {
  hipLaunchKernelGGL((ln_fwd_kernel<T, NV>), dim3((rows + kFwdRows - 1) / kFwdRows),
                     dim3(kLnThreads), 0, s, (const T*)x, g, b, eps, rows, width, (T*)xn,
                     (T*)xn_lo, mean, rstd);
  return hipGetLastError();
}

template <typename T>
hipError_t fwd_t(const void* x, const float* g, const float* b, float eps, int rows, int width,
                 void* xn, void* xn_lo, float* mean, float* rstd, hipStream_t s) {
  const int nv = (width / 8 + kLnThreads - 1) / kLnThreads;
  switch (nv) {
    case 1: return fwd_nv<T, 1>(x, g, b, eps, rows, width, xn, xn_lo, mean, rstd, s);
    case 2: return fwd_nv<T, 2>(x, g, b, eps, rows, width, xn, xn_lo, mean, rstd, s);
    case 3: return fwd_nv<T, 3>(x, g, b, eps, rows, width, xn, xn_lo, mean, rstd, s);
    case 4: return fwd_nv<T, 4>(x, g, b, eps, rows, width, xn, xn_lo, mean, rstd, s);
    case 5: return fwd_nv<T, 5>(x, g, b, eps, rows, width, xn, xn_lo, mean, rstd, s);
    case 6: return fwd_nv<T, 6>(x, g, b, eps, rows, width, xn, xn_lo, mean, rstd, s);
    case 7: return fwd_nv<T, 7>(x, g, b, eps, rows, width, xn, xn_lo, mean, rstd, s);
    default: return fwd_nv<T, 8>(x, g, b, eps, rows, width, xn, xn_lo, mean, rstd, s);
  }
}

template <typename T, int NV>
hipError_t bwd_nv(const void* x, const float* gamma, const float* mean, const float* rstd,
                  const void* dxn, const void* dy, void* dx, float* gp, float* bp, int rows,
                  int width, hipStream_t s) {
  const int nblk = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  // the prefetched row fits in registers up to 3 vectors per thread for
  // bf16 rows, 2 for fp32 rows
  if constexpr (NV <= (sizeof(T) == 2 ? 3 : 2))
    hipLaunchKernelGGL((ln_bwd_kernel<T, NV>), dim3(nblk), dim3(kLnThreads), 0, s,
                       (const T*)x, gamma, mean, rstd, (const T*)dxn, (const T*)dy, (T*)dx, gp, bp,
                       rows,
                       width);
  else
    hipLaunchKernelGGL((ln_bwd_plain_kernel<T, NV>), dim3(nblk), dim3(kLnThreads), 0, s,
                       (const T*)x, gamma, mean, rstd, (const T*)dxn, (const T*)dy, (T*)dx, gp, bp,
                       rows,
                       width);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_t(const void* x, const float* gamma, const float* mean, const float* rstd,
                 const void* dxn, const void* dy, void* dx, float* gp, float* bp, int rows,
                 int width, hipStream_t s) {
  const int nv = (width / 8 + kLnThreads - 1) / kLnThreads;
  switch (nv) {
    case 1: return bwd_nv<T, 1>(x, gamma, mean, rstd, dxn, dy, dx, gp, bp, rows, width, s);
    case 2: return bwd_nv<T, 2>(x, gamma, mean, rstd, dxn, dy, dx, gp, bp, rows, width, s);
    case 3: return bwd_nv<T, 3>(x, gamma, mean, rstd, dxn, dy, dx, gp, bp, rows, width, s);
    case 4: return bwd_nv<T, 4>(x, gamma, mean, rstd, dxn, dy, dx, gp, bp, rows, width, s);
    case 5: return bwd_nv<T, 5>(x, gamma, mean, rstd, dxn, dy, dx, gp, bp, rows, width, s);
    case 6: return bwd_nv<T, 6>(x, gamma, mean, rstd, dxn, dy, dx, gp, bp, rows, width, s);
    case 7: return bwd_nv<T, 7>(x, gamma, mean, rstd, dxn, dy, dx, gp, bp, rows, width, s);
    default: return bwd_nv<T, 8>(x, gamma, mean, rstd, dxn, dy, dx, gp, bp, rows, width, s);
  }
}

}  // namespace

int ln_bwd_rows_per_block() { return kRowsPerBlock; }

hipError_t launch_ln_fwd(int dtype, const void* x, const float* gamma, const float* beta,
                         float eps, int rows, int width, void* xn, void* xn_lo, float* mean,
                         float* rstd, hipStream_t s) {
  if (dtype == 1)
    return fwd_t<bf16_t>(x, gamma, beta, eps, rows, width, xn, xn_lo, mean, rstd, s);
  return fwd_t<float>(x, gamma, beta, eps, rows, width, xn, nullptr, mean, rstd, s);
}

hipError_t launch_ln_bwd(int dtype, const void* x, const float* gamma, const float* mean,
                         const float* rstd, const void* dxn, const void* dy, void* dx,
                         float* gpart, float* bpart, int rows, int width, hipStream_t s) {
  if (dtype == 1)
    return bwd_t<bf16_t>(x, gamma, mean, rstd, dxn, dy, dx, gpart, bpart, rows, width, s);
  return bwd_t<float>(x, gamma, mean, rstd, dxn, dy, dx, gpart, bpart, rows, width, s);
}

hipError_t launch_ln_bwd_reduce(const float* gpart, const float* bpart, int nblk, int width,
                                float* dgamma, float* dbeta, hipStream_t s) {
  hipLaunchKernelGGL(ln_bwd_reduce_kernel, dim3((width + kRedCols - 1) / kRedCols),
                     dim3(kRedCols * kRedGroups), 0, s, gpart, bpart, nblk, width, dgamma, dbeta);
  return hipGetLastError();
}

}  // namespace ptb
