// Fused LAMB optimizer step (MegaScale study guide, ch.2 §2.2 technique
// table, LAMB row: a layer-wise adaptive trust ratio, the method of You et
// al. 2020, which MegaScale uses to enlarge the batch).  Each parameter
// tensor is one "layer": its update u is scaled by ||w|| / ||u||.
//
// The trust ratio needs the norm of the whole u before any w can change, so
// the step is two streaming passes plus a tiny combine:
//   pass A   reads w, g, m, v; writes m' and v'; each workgroup writes its
//            partial sums of w^2 and u^2               (22 bytes/param, bf16 g)
//   finalize one workgroup per tensor adds that tensor's partials in fp64, in
//            block order (deterministic), and stores r = ||w||/||u|| (r = 1
//            when a norm is 0)
//   pass B   reads w, m', v'; recomputes u with the same instructions as
//            pass A; writes w - lr * r * u                (16 bytes/param)
//            and, when asked, a bf16 copy of the new w for the next
//            forward                                      (+2 bytes/param)
// The sharded form (ZeRO-2: each data-parallel rank owns a contiguous
// element range of every tensor) splits the step at the norms: pass A plus
// a finalize that stores the shard's fp64 sums of w^2 and u^2 per tensor;
// the caller adds those over the ranks (an all-reduce of 2 doubles per
// tensor); then the ratios come from the summed norms and pass B runs on
// the shard.
// All tensors of a call share one launch per pass (a kernel-argument table
// of up to 16 tensors; a workgroup finds its tensor from the block ranges).
// Each thread moves 16-byte vectors (4 fp32) and keeps 4 of them in flight
// per array.  Every stream is touched once per pass, so loads and stores
// carry the non-temporal hint (measured on this access mix: about 5.3 TB/s
// without it, 5.7-6.0 TB/s with it).
#include "common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr int kLambThreads = 256;
constexpr int kLambUnroll = 4;
constexpr int kLambChunk = kLambThreads * 4 * kLambUnroll;  // elements per workgroup

__device__ __forceinline__ float4 ld_nt(const float* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_nt(float* p, float4 v) {
  const f32x4_t t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t*>(p));
}
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld_nt(const bf16_t* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st_nt(bf16_t* p, uint2 v) {
  const u32x2_t t = {v.x, v.y};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x2_t*>(p));
}

__device__ __forceinline__ int find_tensor(const LambBatch& b, int blk) {
  int t = 0;
#pragma unroll
  for (int i = 1; i < kLambMaxTensors; ++i)
    if (i < b.ntensors && blk >= b.blk_start[i]) t = i;
  return t;
}

template <typename G> struct GradLoad;
template <> struct GradLoad<bf16_t> {
  static __device__ __forceinline__ float4 ld4(const void* p, int64_t i) {
    const uint2 u = ld_nt(static_cast<const bf16_t*>(p) + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
  static __device__ __forceinline__ float ld1(const void* p, int64_t i) {
    return bf2f(static_cast<const bf16_t*>(p)[i]);
  }
};
template <> struct GradLoad<float> {
  static __device__ __forceinline__ float4 ld4(const void* p, int64_t i) {
    return ld_nt(static_cast<const float*>(p) + i);
  }
  static __device__ __forceinline__ float ld1(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
};

// The update direction of one element, identical in both passes.
__device__ __forceinline__ float lamb_u(float w, float m, float v, float wd,
                                        const LambHyper& hp) {
  const float mh = m / hp.bc1;
  const float vh = v / hp.bc2;
  return mh / (sqrtf(vh) + hp.eps) + wd * w;
}

// Pass A over one workgroup's chunk of tensor t; returns this thread's
// partial sums of w^2 and u^2.
template <typename G>
__device__ __forceinline__ void pass_a_chunk(const LambBatch& b, const LambHyper& hp, int t,
                                             int64_t base, float& sw, float& su) {
  const int64_t n = b.n[t];
  float* w = b.w[t];
  float* m = b.m[t];
  float* v = b.v[t];
  const void* g = b.g[t];
  const float wd = b.wd[t];
  const float c1 = 1.f - hp.beta1, c2 = 1.f - hp.beta2;
  if (base + kLambChunk <= n) {
    float4 wv[kLambUnroll], mv[kLambUnroll], vv[kLambUnroll], gv[kLambUnroll];
#pragma unroll
    for (int u = 0; u < kLambUnroll; ++u) {
      const int64_t i = base + (int64_t)(u * kLambThreads + threadIdx.x) * 4;
      wv[u] = ld_nt(w + i);
      mv[u] = ld_nt(m + i);
      vv[u] = ld_nt(v + i);
      gv[u] = GradLoad<G>::ld4(g, i);
    }
#pragma unroll
    for (int u = 0; u < kLambUnroll; ++u) {
      const int64_t i = base + (int64_t)(u * kLambThreads + threadIdx.x) * 4;
      float ww[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
      float mm[4] = {mv[u].x, mv[u].y, mv[u].z, mv[u].w};
      float vs[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
      const float gg[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mm[e] = hp.beta1 * mm[e] + c1 * gg[e];
        vs[e] = hp.beta2 * vs[e] + c2 * gg[e] * gg[e];
        const float uu = lamb_u(ww[e], mm[e], vs[e], wd, hp);
        sw += ww[e] * ww[e];
        su += uu * uu;
      }
      st_nt(m + i, make_float4(mm[0], mm[1], mm[2], mm[3]));
      st_nt(v + i, make_float4(vs[0], vs[1], vs[2], vs[3]));
    }
  } else {
    for (int64_t i = base + threadIdx.x; i < min(n, base + kLambChunk); i += kLambThreads) {
      const float gg = GradLoad<G>::ld1(g, i);
      const float mm = hp.beta1 * m[i] + c1 * gg;
      const float vs = hp.beta2 * v[i] + c2 * gg * gg;
      const float ww = w[i];
      const float uu = lamb_u(ww, mm, vs, wd, hp);
      m[i] = mm;
      v[i] = vs;
      sw += ww * ww;
      su += uu * uu;
    }
  }
}

__global__ __launch_bounds__(kLambThreads) void lamb_pass_a(LambBatch b, LambHyper hp,
                                                            float* __restrict__ partials) {
  __shared__ float red[kLambThreads / 64];
  const int blk = blockIdx.x;
  const int t = find_tensor(b, blk);
  const int64_t base = (int64_t)(blk - b.blk_start[t]) * kLambChunk;
  float sw = 0.f, su = 0.f;
  if (b.gdt[t] == 1)
    pass_a_chunk<bf16_t>(b, hp, t, base, sw, su);
  else
    pass_a_chunk<float>(b, hp, t, base, sw, su);
  sw = block_sum<kLambThreads / 64>(sw, red);
  su = block_sum<kLambThreads / 64>(su, red);
  if (threadIdx.x == 0) {
    partials[2 * blk] = sw;
    partials[2 * blk + 1] = su;
  }
}

// One workgroup of 1024 threads per tensor; thread i adds partials i,
// i + 1024, ... in fp64, then the 16 wave sums are added in wave order.
constexpr int kFinThreads = 1024;
__device__ __forceinline__ void tensor_sums(const LambBatch& b, const float* __restrict__ partials,
                                            int t, double& W, double& U) {
  __shared__ double red[2][kFinThreads / 64];
  double sw = 0.0, su = 0.0;
#pragma unroll 4
  for (int blk = b.blk_start[t] + threadIdx.x; blk < b.blk_start[t + 1]; blk += kFinThreads) {
    const float2 p = *reinterpret_cast<const float2*>(partials + 2 * blk);
    sw += (double)p.x;
    su += (double)p.y;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sw += __shfl_xor(sw, o, 64);
    su += __shfl_xor(su, o, 64);
  }
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][wid] = sw; red[1][wid] = su; }
  __syncthreads();
  W = 0.0;
  U = 0.0;
  if (threadIdx.x == 0)
    for (int i = 0; i < kFinThreads / 64; ++i) { W += red[0][i]; U += red[1][i]; }
}

__device__ __forceinline__ float trust_ratio(double W, double U) {
  return (W > 0.0 && U > 0.0) ? (float)(sqrt(W) / sqrt(U)) : 1.0f;
}

__global__ __launch_bounds__(kFinThreads) void lamb_finalize(LambBatch b,
                                                             const float* __restrict__ partials,
                                                             float* __restrict__ ratios,
                                                             float* __restrict__ ratios_out) {
  double W, U;
  tensor_sums(b, partials, blockIdx.x, W, U);
  if (threadIdx.x == 0) {
    const float r = trust_ratio(W, U);
    ratios[blockIdx.x] = r;
    if (ratios_out != nullptr) ratios_out[blockIdx.x] = r;
  }
}

// Sharded step, first half: this shard's sum of w^2 and u^2 per tensor.
__global__ __launch_bounds__(kFinThreads) void lamb_finalize_norms(
    LambBatch b, const float* __restrict__ partials, double* __restrict__ norms) {
  double W, U;
  tensor_sums(b, partials, blockIdx.x, W, U);
  if (threadIdx.x == 0) {
    norms[2 * blockIdx.x] = W;
    norms[2 * blockIdx.x + 1] = U;
  }
}

// Sharded step, second half: the ratios from the norms summed over shards.
__global__ __launch_bounds__(64) void lamb_ratios_from_norms(int n, const double* __restrict__ norms,
                                                             float* __restrict__ ratios,
                                                             float* __restrict__ ratios_out) {
  const int t = threadIdx.x;
  if (t >= n) return;
  const float r = trust_ratio(norms[2 * t], norms[2 * t + 1]);
  ratios[t] = r;
  if (ratios_out != nullptr) ratios_out[t] = r;
}

__global__ __launch_bounds__(kLambThreads) void lamb_pass_b(LambBatch b, LambHyper hp,
                                                            const float* __restrict__ ratios) {
  const int blk = blockIdx.x;
  const int t = find_tensor(b, blk);
  const int64_t n = b.n[t];
  const int64_t base = (int64_t)(blk - b.blk_start[t]) * kLambChunk;
  float* w = b.w[t];
  const float* m = b.m[t];
  const float* v = b.v[t];
  bf16_t* wc = static_cast<bf16_t*>(b.wc[t]);
  const float wd = b.wd[t];
  const float step = hp.lr * ratios[t];
  if (base + kLambChunk <= n) {
    float4 wv[kLambUnroll], mv[kLambUnroll], vv[kLambUnroll];
#pragma unroll
    for (int u = 0; u < kLambUnroll; ++u) {
      const int64_t i = base + (int64_t)(u * kLambThreads + threadIdx.x) * 4;
      wv[u] = ld_nt(w + i);
      mv[u] = ld_nt(m + i);
      vv[u] = ld_nt(v + i);
    }
#pragma unroll
    for (int u = 0; u < kLambUnroll; ++u) {
      const int64_t i = base + (int64_t)(u * kLambThreads + threadIdx.x) * 4;
      float4 o;
      o.x = wv[u].x - step * lamb_u(wv[u].x, mv[u].x, vv[u].x, wd, hp);
      o.y = wv[u].y - step * lamb_u(wv[u].y, mv[u].y, vv[u].y, wd, hp);
      o.z = wv[u].z - step * lamb_u(wv[u].z, mv[u].z, vv[u].z, wd, hp);
      o.w = wv[u].w - step * lamb_u(wv[u].w, mv[u].w, vv[u].w, wd, hp);
      st_nt(w + i, o);
      if (wc != nullptr) st_nt(wc + i, make_uint2(pack_bf2(o.x, o.y), pack_bf2(o.z, o.w)));
    }
  } else {
    for (int64_t i = base + threadIdx.x; i < min(n, base + kLambChunk); i += kLambThreads) {
      const float o = w[i] - step * lamb_u(w[i], m[i], v[i], wd, hp);
      w[i] = o;
      if (wc != nullptr) wc[i] = f2bf(o);
    }
  }
}

}  // namespace

int64_t lamb_blocks_for(int64_t n) { return (n + kLambChunk - 1) / kLambChunk; }

hipError_t launch_lamb(const LambBatch& b, const LambHyper& hp, float* partials, float* ratios,
                       float* ratios_out, hipStream_t s) {
  const int nblk = b.blk_start[b.ntensors];
  hipLaunchKernelGGL(lamb_pass_a, dim3(nblk), dim3(kLambThreads), 0, s, b, hp, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lamb_finalize, dim3(b.ntensors), dim3(kFinThreads), 0, s, b,
                     (const float*)partials, ratios, ratios_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lamb_pass_b, dim3(nblk), dim3(kLambThreads), 0, s, b, hp,
                     (const float*)ratios);
  return hipGetLastError();
}

hipError_t launch_lamb_norms(const LambBatch& b, const LambHyper& hp, float* partials,
                             double* norms, hipStream_t s) {
  const int nblk = b.blk_start[b.ntensors];
  hipLaunchKernelGGL(lamb_pass_a, dim3(nblk), dim3(kLambThreads), 0, s, b, hp, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lamb_finalize_norms, dim3(b.ntensors), dim3(kFinThreads), 0, s, b,
                     (const float*)partials, norms);
  return hipGetLastError();
}

hipError_t launch_lamb_apply(const LambBatch& b, const LambHyper& hp, const double* norms,
                             float* ratios, float* ratios_out, hipStream_t s) {
  hipLaunchKernelGGL(lamb_ratios_from_norms, dim3(1), dim3(64), 0, s, b.ntensors, norms, ratios,
                     ratios_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nblk = b.blk_start[b.ntensors];
  hipLaunchKernelGGL(lamb_pass_b, dim3(nblk), dim3(kLambThreads), 0, s, b, hp,
                     (const float*)ratios);
  return hipGetLastError();
}

}  // namespace ptb
