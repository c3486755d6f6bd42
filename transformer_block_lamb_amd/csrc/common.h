// Shared device helpers for the gfx950 kernels: vector types, bf16
// conversion, buffer resources with hardware out-of-range zero fill, MFMA
// wrappers and wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptb {

typedef unsigned short bf16_t;  // storage type of bfloat16 values
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf2f(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round-to-nearest-even via the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

// Element type traits: load/store one element as fp32.
template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static __device__ __forceinline__ float ld_rounded(float v) { return v; }  // v as stored
};
template <> struct Elt<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }
  static __device__ __forceinline__ float ld_rounded(float v) { return bf2f(f2bf(v)); }
};

// 8 consecutive elements of a row as fp32.
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float (&o)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[8]) {
    uint4 u;
    u.x = pack_bf2(v[0], v[1]); u.y = pack_bf2(v[2], v[3]);
    u.z = pack_bf2(v[4], v[5]); u.w = pack_bf2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = u;
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float (&o)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// ---------------------------------------------------------------- buffers
// A raw buffer resource: loads whose byte offset lies at or beyond
// `bytes` return zeros (hardware range check), so tile loaders mask a ragged
// edge by steering the offset out of range instead of branching.
// LDS (address space 3) pointer types for the LDS-bound buffer loads and
// the transposing LDS reads.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBufferFlags = 0x00020000;  // gfx9 data format word of the descriptor

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferFlags);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

// ---------------------------------------------------------------- MFMA
// D = A * B + C for a 32x32 output block with K = 16.  Lane l supplies
// A[l%32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l%32]; it receives
// D[8*(r/4) + 4*(l/32) + r%4][l%32] in element r of the result.
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// Row of the 32x32 MFMA output held in element r of lane l.
__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// 8x8 transpose of bf16 held as 8 rows of uint4 (row i = 8 values).
// out[j] element i == in[i] element j.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
  uint32_t w[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    w[i][0] = in[i].x; w[i][1] = in[i].y; w[i][2] = in[i].z; w[i][3] = in[i].w;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t o[4];
    const int src = j >> 1;      // dword holding column j in each input row
    const bool hi = (j & 1);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t a = w[2 * p][src], b = w[2 * p + 1][src];
      o[p] = hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    out[j] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
// Sum over a workgroup of `nwaves` waves; `red` is LDS of >= nwaves floats.
// Every thread receives the total.  Contains two barriers.
template <int NWAVES>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) t += red[i];
  __syncthreads();
  return t;
}

// Two independent sums over a workgroup at once (one LDS exchange, two
// barriers instead of four); `red` is LDS of >= 2 * NWAVES floats.
template <int NWAVES>
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) {
    red[wid] = a;
    red[NWAVES + wid] = b;
  }
  __syncthreads();
  float ta = 0.f, tb = 0.f;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    ta += red[i];
    tb += red[NWAVES + i];
  }
  __syncthreads();
  a = ta;
  b = tb;
}

// ---------------------------------------------------------------- GeLU
// erf by the rational approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (absolute error <= 1.5e-7), written
// inline so that epilogues holding hundreds of accumulators make no calls.
// The reciprocal and the exponential use the hardware approximations
// (v_rcp_f32, v_exp_f32: about one ulp), far inside the formula's own error.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float y = 1.0f - poly * __builtin_amdgcn_exp2f(-1.4426950408889634f * ax * ax);
  return copysignf(y, x);
}
// Exact GeLU f * Phi(f) and its derivative Phi(f) + f * phi(f).
__device__ __forceinline__ float gelu_f(float f) {
  return 0.5f * f * (1.0f + erf_as(f * 0.70710678118654752f));
}
// (The derivative evaluates exp(-f^2 / 2) once: the erf formula at
// f / sqrt(2) and the normal density both use it.)
__device__ __forceinline__ float gelu_grad_f(float f) {
  const float x = f * 0.70710678118654752f, ax = fabsf(x);
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * ax * ax);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float erf = copysignf(1.0f - poly * e, x);
  return 0.5f * (1.0f + erf) + f * (0.39894228040143268f * e);
}

}  // namespace ptb
