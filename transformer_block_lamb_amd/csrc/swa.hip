// Causal sliding-window attention (MegaScale study guide, ch.2 §2.2 technique
// table, SWA row: every token attends to a fixed window of w tokens, so the
// cost is O(s*w) instead of O(s*s)).  Key j is visible to query i of the same
// sequence iff 0 <= i - j < w; scores are scaled by 1/sqrt(d).
//
// bf16 path, one workgroup = 4 waves, every wave owns 32 queries (forward,
// dQ) or 32 keys (dK/dV) and computes 32x32 blocks with
// v_mfma_f32_32x32x16_bf16:
//   * forward: a block of 128 queries walks only the 64-key tiles that
//     intersect its band; each wave skips tiles outside its own band and
//     masks only tiles that cross the band edges.  Scores are computed
//     transposed (S^T = K Q^T) so that each lane holds 16 scores of ONE
//     query: the online softmax (running max and sum, base-2 exponent) then
//     needs a single lane exchange, and the probabilities already sit in
//     the B-operand layout of O^T += V^T P^T (keys reordered inside the K=16
//     step, the same order used to read V^T from LDS).  V is transposed in
//     registers (8x8 blocks) on its way into LDS.  The log-sum-exp of each
//     query is written for the backward.
//   * backward (FlashAttention-2 style, no atomics, deterministic):
//     D_i = dO_i . O_i; then one kernel per 128-key block accumulates dK and
//     dV over the query tiles of the band (S = Q K^T, P = exp(S - lse),
//     dP = dO V^T, dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS), and one
//     kernel per 128-query block accumulates dQ^T += K^T dS^T with the
//     transposed formulation of the forward.
// fp32 path: one thread per query (or key) looping over its window; it serves
// the fp32 workload only.
#include "common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBQ = 128, kBKV = 64, kSwaThreads = 256;
constexpr int kTLD = kBKV + 8;  // row stride (elements) of transposed LDS tiles

__device__ __forceinline__ bf16x8_t ld_frag(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}
// A-operand fragment of a transposed tile whose K index is the reordered
// key/query order used for probabilities held in MFMA output layout: lane l
// takes elements [base + 4*(l/32) + 0..3] and [base + 8 + 4*(l/32) + 0..3].
__device__ __forceinline__ bf16x8_t ld_frag_reordered(const bf16_t* row, int lane) {
  const bf16_t* p = row + 4 * (lane >> 5);
  const uint2 lo = *reinterpret_cast<const uint2*>(p);
  const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
  return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
__device__ __forceinline__ bf16x8_t pack8(const float* v) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]),
                                                  pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])));
}
__device__ __forceinline__ bool visible(int i, int j, int w) { return j <= i && i - j < w; }

// Register-staged copies of one 64-row tile, so the loads of the next tile
// can be issued before the current one is consumed: load() issues every
// global load of this thread's share at once, store() writes it to LDS.
// RowTile: rows [r0, r0 + 64) x D into LDS row-major (stride D + 8); thread
// t owns 16-byte chunks t, t + 256, ... (D / 32 of them).
template <int D>
struct RowTile {
  static constexpr int CH = D / 8, N = kBKV * CH / kSwaThreads;
  static_assert(N * kSwaThreads == kBKV * CH, "whole chunks per thread");
  uint4 v[N];
  __device__ __forceinline__ void load(const bf16_t* src, int64_t ld, int r0, int seq) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + i * kSwaThreads, r = c / CH, cc = c - r * CH;
      v[i] = r0 + r < seq ? *reinterpret_cast<const uint4*>(src + (int64_t)(r0 + r) * ld + cc * 8)
                          : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16_t* dst) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = threadIdx.x + i * kSwaThreads, r = c / CH, cc = c - r * CH;
      *reinterpret_cast<uint4*>(dst + r * (D + 8) + cc * 8) = v[i];
    }
  }
};
// RowTileT: the same rows stored transposed, dst[dim][row] with stride kTLD;
// thread t < D owns the 8-row x 8-dim block (rows 8 (t & 7), dims 8 (t >> 3))
// and transposes it in registers.
template <int D>
struct RowTileT {
  uint4 v[8];
  __device__ __forceinline__ void load(const bf16_t* src, int64_t ld, int r0, int seq) {
    const int t = threadIdx.x, rb = t & 7, db = t >> 3;
    if (t < D) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = r0 + rb * 8 + i;
        v[i] = r < seq ? *reinterpret_cast<const uint4*>(src + (int64_t)r * ld + db * 8)
                       : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t* dst) const {
    const int t = threadIdx.x, rb = t & 7, db = t >> 3;
    if (t < D) {
      uint4 out[8];
      transpose8x8(v, out);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd)
        *reinterpret_cast<uint4*>(dst + (db * 8 + dd) * kTLD + rb * 8) = out[dd];
    }
  }
};

template <class Tile>
__device__ __forceinline__ void stage(bf16_t* dst, const bf16_t* src, int64_t ld, int r0, int seq) {
  Tile t;
  t.load(src, ld, r0, seq);
  t.store(dst);
}

// ------------------------------------------------------------------ forward
// Loads this lane's B-operand fragments of one token row (8 consecutive
// dims per K=16 step): row `r` of a token-major matrix, zero beyond `seq`.
template <int D>
__device__ __forceinline__ void load_row_frags(bf16x8_t (&f)[D / 16], const bf16_t* src,
                                               int64_t ld, int r, int seq, int lane) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < seq) v = *reinterpret_cast<const uint4*>(src + (int64_t)r * ld + ks * 16 + (lane >> 5) * 8);
    f[ks] = __builtin_bit_cast(bf16x8_t, v);
  }
}

// SPLIT: q and k also come as bf16 residuals (qk_lo [T, 2A], leading
// dimension ldl); every score is q_hi.k_hi + q_hi.k_lo + q_lo.k_hi, which
// keeps the scores at fp32-level accuracy.
template <int D, bool SPLIT>
__global__ __launch_bounds__(kSwaThreads) void swa_fwd_mfma(const bf16_t* __restrict__ qkv,
                                                            int64_t ldq,
                                                            const bf16_t* __restrict__ qk_lo,
                                                            int64_t ldl, bf16_t* __restrict__ out,
                                                            int64_t ldo, float* __restrict__ lse,
                                                            int S, int H, int W, float sl2) {
  constexpr int KLD = D + 8;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[kBKV * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t Ks_lo[SPLIT ? kBKV * KLD : 8];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[D * kTLD];
  const int h = blockIdx.y, b = blockIdx.z;
  const int A = H * D;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q0 = blockIdx.x * kBQ;
  const int qw = q0 + wave * 32;
  const int qi = qw + (lane & 31);
  const bf16_t* base = qkv + (int64_t)b * S * ldq;
  const bf16_t* Qp = base + h * D;
  const bf16_t* Kp = base + A + h * D;
  const bf16_t* Vp = base + 2 * A + h * D;
  const bf16_t* lo_base = SPLIT ? qk_lo + (int64_t)b * S * ldl : nullptr;

  bf16x8_t qf[D / 16], qf_lo[D / 16];
  load_row_frags<D>(qf, Qp, ldq, qi, S, lane);
  if (SPLIT) load_row_frags<D>(qf_lo, lo_base + h * D, ldl, qi, S, lane);
  f32x16_t o[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int qlast = min(q0 + kBQ, S) - 1;
  const int kt_lo = max(0, q0 - W + 1) / kBKV, kt_hi = qlast / kBKV;
  const bool wave_live = qw < S;
  // tile kt + 1 is loaded into registers while tile kt is multiplied
  RowTile<D> kreg, klreg;
  RowTileT<D> vreg;
  const bf16_t* Klp = SPLIT ? lo_base + A + h * D : nullptr;
  kreg.load(Kp, ldq, kt_lo * kBKV, S);
  if (SPLIT) klreg.load(Klp, ldl, kt_lo * kBKV, S);
  vreg.load(Vp, ldq, kt_lo * kBKV, S);
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int j0 = kt * kBKV;
    __syncthreads();
    kreg.store(Ks);
    if (SPLIT) klreg.store(Ks_lo);
    vreg.store(Vt);
    __syncthreads();
    if (kt < kt_hi) {
      kreg.load(Kp, ldq, j0 + kBKV, S);
      if (SPLIT) klreg.load(Klp, ldl, j0 + kBKV, S);
      vreg.load(Vp, ldq, j0 + kBKV, S);
    }
    if (!wave_live || j0 > qw + 31 || j0 + kBKV - 1 < qw - W + 1) continue;
    const bool full = (j0 + kBKV - 1 <= qw) && (qw + 31 - j0 < W) && (j0 + kBKV <= S);
    f32x16_t st[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kh][r] = 0.f;
      const int fo = (kh * 32 + (lane & 31)) * KLD + (lane >> 5) * 8;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8_t kf = ld_frag(Ks + fo + ks * 16);
        st[kh] = mfma32(kf, qf[ks], st[kh]);
        if (SPLIT) {
          st[kh] = mfma32(kf, qf_lo[ks], st[kh]);
          st[kh] = mfma32(ld_frag(Ks_lo + fo + ks * 16), qf[ks], st[kh]);
        }
      }
    }
    float mblk = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float sv = st[kh][r] * sl2;
        if (!full) {
          const int j = j0 + kh * 32 + mfma32_row(r, lane);
          if (!(visible(qi, j, W) && j < S)) sv = -INFINITY;
        }
        st[kh][r] = sv;
        mblk = fmaxf(mblk, sv);
      }
    mblk = fmaxf(mblk, __shfl_xor(mblk, 32, 64));
    const float m_new = fmaxf(m_run, mblk);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
    m_run = m_new;
    float p[2][16];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[kh][r] = exp2f(st[kh][r] - m_use);
        l_run += p[kh][r];
      }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16x8_t pb = pack8(&p[kh][hf * 8]);
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
          const bf16_t* vr = Vt + (mb * 32 + (lane & 31)) * kTLD + kh * 32 + hf * 16;
          o[mb] = mfma32(ld_frag_reordered(vr, lane), pb, o[mb]);
        }
      }
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qi < S) {
    const float inv = 1.0f / l_tot;
    bf16_t* orow = out + ((int64_t)b * S + qi) * ldo + h * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * (lane >> 5);
        uint2 u;
        u.x = pack_bf2(o[mb][4 * g] * inv, o[mb][4 * g + 1] * inv);
        u.y = pack_bf2(o[mb][4 * g + 2] * inv, o[mb][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d0) = u;
      }
    if (lane < 32) lse[((int64_t)b * H + h) * S + qi] = (m_run + log2f(l_tot)) * kLn2;
  }
}

// ------------------------------------------------------------------ D = rowsum(dO * O)
// One thread per (batch, head, query); the head's D values of dO and O move
// as 8-element vectors (D is a multiple of 8).
template <typename T>
__global__ __launch_bounds__(256) void swa_rowdot(const T* __restrict__ d_o, int64_t ld_do,
                                                  const T* __restrict__ o, int64_t ldo,
                                                  float* __restrict__ dvec, int B, int S, int H,
                                                  int D) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, h, i) flattened
  if (idx >= (int64_t)B * H * S) return;
  const int i = idx % S;
  const int h = (idx / S) % H;
  const int b = idx / ((int64_t)S * H);
  const int64_t t = (int64_t)b * S + i;
  const T* a = d_o + t * ld_do + h * D;
  const T* c = o + t * ldo + h * D;
  float s = 0.f;
  for (int k = 0; k < D; k += 8) {
    float va[8], vc[8];
    Vec8<T>::load(a + k, va);
    Vec8<T>::load(c + k, vc);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += va[e] * vc[e];
  }
  dvec[idx] = s;
}

// ------------------------------------------------------------------ dK, dV
template <int D, bool SPLIT>
__global__ __launch_bounds__(kSwaThreads) void swa_bwd_dkdv_mfma(
    const bf16_t* __restrict__ qkv, int64_t ldq, const bf16_t* __restrict__ qk_lo, int64_t ldl,
    const bf16_t* __restrict__ d_o, int64_t ld_do,
    const float* __restrict__ lse, const float* __restrict__ dvec, bf16_t* __restrict__ dqkv,
    int64_t ldd, int S, int H, int W, float sl2, float scale) {
  constexpr int KLD = D + 8;
  __shared__ __attribute__((aligned(16))) bf16_t Qs[kBKV * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t Qs_lo[SPLIT ? kBKV * KLD : 8];
  __shared__ __attribute__((aligned(16))) bf16_t dOs[kBKV * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t Qt[D * kTLD];
  __shared__ __attribute__((aligned(16))) bf16_t dOt[D * kTLD];
  __shared__ __attribute__((aligned(16))) float lse_s[kBKV];
  __shared__ __attribute__((aligned(16))) float dv_s[kBKV];
  const int h = blockIdx.y, b = blockIdx.z;
  const int A = H * D;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k0 = blockIdx.x * kBQ;
  const int kw = k0 + wave * 32;
  const int kj = kw + (lane & 31);
  const bf16_t* base = qkv + (int64_t)b * S * ldq;
  const bf16_t* Qp = base + h * D;
  const bf16_t* Kp = base + A + h * D;
  const bf16_t* Vp = base + 2 * A + h * D;
  const bf16_t* dOp = d_o + (int64_t)b * S * ld_do + h * D;
  const float* lse_b = lse + ((int64_t)b * H + h) * S;
  const float* dv_b = dvec + ((int64_t)b * H + h) * S;
  const bf16_t* lo_base = SPLIT ? qk_lo + (int64_t)b * S * ldl : nullptr;

  bf16x8_t kf[D / 16], vf[D / 16], kf_lo[D / 16];
  load_row_frags<D>(kf, Kp, ldq, kj, S, lane);
  load_row_frags<D>(vf, Vp, ldq, kj, S, lane);
  if (SPLIT) load_row_frags<D>(kf_lo, lo_base + A + h * D, ldl, kj, S, lane);
  f32x16_t dk[D / 32], dv[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[mb][r] = 0.f; dv[mb][r] = 0.f; }

  const int klast = min(k0 + kBQ, S) - 1;
  const int qt_lo = k0 / kBKV, qt_hi = min(S - 1, klast + W - 1) / kBKV;
  const bool wave_live = kw < S;
  for (int qt = qt_lo; qt <= qt_hi; ++qt) {
    const int i0 = qt * kBKV;
    __syncthreads();
    // each array's loads in flight at once, then its LDS stores (one array
    // at a time: this kernel holds dK and dV for 128 keys in registers)
    stage<RowTile<D>>(Qs, Qp, ldq, i0, S);
    if (SPLIT) stage<RowTile<D>>(Qs_lo, lo_base + h * D, ldl, i0, S);
    stage<RowTile<D>>(dOs, dOp, ld_do, i0, S);
    stage<RowTileT<D>>(Qt, Qp, ldq, i0, S);
    stage<RowTileT<D>>(dOt, dOp, ld_do, i0, S);
    if (threadIdx.x < kBKV) {
      const int i = i0 + threadIdx.x;
      lse_s[threadIdx.x] = i < S ? lse_b[i] * kLog2e : 0.f;
      dv_s[threadIdx.x] = i < S ? dv_b[i] : 0.f;
    }
    __syncthreads();
    if (!wave_live || i0 > kw + 31 + W - 1 || i0 + kBKV - 1 < kw) continue;
    const bool full = (i0 >= kw + 31) && (i0 + kBKV - 1 - kw < W) && (i0 + kBKV <= S);
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      f32x16_t s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
      const int fo = (qh * 32 + (lane & 31)) * KLD + (lane >> 5) * 8;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8_t qa = ld_frag(Qs + fo + ks * 16);
        s = mfma32(qa, kf[ks], s);
        if (SPLIT) {
          s = mfma32(qa, kf_lo[ks], s);
          s = mfma32(ld_frag(Qs_lo + fo + ks * 16), kf[ks], s);
        }
        dp = mfma32(ld_frag(dOs + fo + ks * 16), vf[ks], dp);
      }
      float p[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rb = qh * 32 + 8 * g + 4 * (lane >> 5);
        const float4 l4 = *reinterpret_cast<const float4*>(lse_s + rb);
        const float4 d4 = *reinterpret_cast<const float4*>(dv_s + rb);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pv = exp2f(s[r] * sl2 - lv[e]);
          if (!full) {
            const int i = i0 + rb + e;
            if (!(visible(i, kj, W) && i < S)) pv = 0.f;
          }
          p[r] = pv;
          ds[r] = pv * (dp[r] - dd[e]);
        }
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16x8_t pb = pack8(&p[hf * 8]);
        const bf16x8_t db = pack8(&ds[hf * 8]);
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
          const int ro = (mb * 32 + (lane & 31)) * kTLD + qh * 32 + hf * 16;
          dv[mb] = mfma32(ld_frag_reordered(dOt + ro, lane), pb, dv[mb]);
          dk[mb] = mfma32(ld_frag_reordered(Qt + ro, lane), db, dk[mb]);
        }
      }
    }
  }
  if (kj < S) {
    bf16_t* row = dqkv + ((int64_t)b * S + kj) * ldd + h * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * (lane >> 5);
        uint2 uk, uv;
        uk.x = pack_bf2(dk[mb][4 * g] * scale, dk[mb][4 * g + 1] * scale);
        uk.y = pack_bf2(dk[mb][4 * g + 2] * scale, dk[mb][4 * g + 3] * scale);
        uv.x = pack_bf2(dv[mb][4 * g], dv[mb][4 * g + 1]);
        uv.y = pack_bf2(dv[mb][4 * g + 2], dv[mb][4 * g + 3]);
        *reinterpret_cast<uint2*>(row + A + d0) = uk;
        *reinterpret_cast<uint2*>(row + 2 * A + d0) = uv;
      }
  }
}

// ------------------------------------------------------------------ dQ
template <int D, bool SPLIT>
__global__ __launch_bounds__(kSwaThreads) void swa_bwd_dq_mfma(
    const bf16_t* __restrict__ qkv, int64_t ldq, const bf16_t* __restrict__ qk_lo, int64_t ldl,
    const bf16_t* __restrict__ d_o, int64_t ld_do,
    const float* __restrict__ lse, const float* __restrict__ dvec, bf16_t* __restrict__ dqkv,
    int64_t ldd, int S, int H, int W, float sl2, float scale) {
  constexpr int KLD = D + 8;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[kBKV * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t Ks_lo[SPLIT ? kBKV * KLD : 8];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[kBKV * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t Kt[D * kTLD];
  const int h = blockIdx.y, b = blockIdx.z;
  const int A = H * D;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q0 = blockIdx.x * kBQ;
  const int qw = q0 + wave * 32;
  const int qi = qw + (lane & 31);
  const bf16_t* base = qkv + (int64_t)b * S * ldq;
  const bf16_t* Qp = base + h * D;
  const bf16_t* Kp = base + A + h * D;
  const bf16_t* Vp = base + 2 * A + h * D;
  const bf16_t* dOp = d_o + (int64_t)b * S * ld_do + h * D;
  const bf16_t* lo_base = SPLIT ? qk_lo + (int64_t)b * S * ldl : nullptr;

  bf16x8_t qf[D / 16], of[D / 16], qf_lo[D / 16];
  load_row_frags<D>(qf, Qp, ldq, qi, S, lane);
  load_row_frags<D>(of, dOp, ld_do, qi, S, lane);
  if (SPLIT) load_row_frags<D>(qf_lo, lo_base + h * D, ldl, qi, S, lane);
  const float lse2 = qi < S ? lse[((int64_t)b * H + h) * S + qi] * kLog2e : 0.f;
  const float di = qi < S ? dvec[((int64_t)b * H + h) * S + qi] : 0.f;
  f32x16_t dq[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[mb][r] = 0.f;

  const int qlast = min(q0 + kBQ, S) - 1;
  const int kt_lo = max(0, q0 - W + 1) / kBKV, kt_hi = qlast / kBKV;
  const bool wave_live = qw < S;
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int j0 = kt * kBKV;
    __syncthreads();
    {  // every load of the tile in flight at once, then the LDS stores
      RowTile<D> k, kl, v;
      RowTileT<D> kt_;
      k.load(Kp, ldq, j0, S);
      if (SPLIT) kl.load(lo_base + A + h * D, ldl, j0, S);
      v.load(Vp, ldq, j0, S);
      kt_.load(Kp, ldq, j0, S);
      k.store(Ks);
      if (SPLIT) kl.store(Ks_lo);
      v.store(Vs);
      kt_.store(Kt);
    }
    __syncthreads();
    if (!wave_live || j0 > qw + 31 || j0 + kBKV - 1 < qw - W + 1) continue;
    const bool full = (j0 + kBKV - 1 <= qw) && (qw + 31 - j0 < W) && (j0 + kBKV <= S);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      f32x16_t st, dpt;
#pragma unroll
      for (int r = 0; r < 16; ++r) { st[r] = 0.f; dpt[r] = 0.f; }
      const int fo = (kh * 32 + (lane & 31)) * KLD + (lane >> 5) * 8;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8_t ka = ld_frag(Ks + fo + ks * 16);
        st = mfma32(ka, qf[ks], st);
        if (SPLIT) {
          st = mfma32(ka, qf_lo[ks], st);
          st = mfma32(ld_frag(Ks_lo + fo + ks * 16), qf[ks], st);
        }
        dpt = mfma32(ld_frag(Vs + fo + ks * 16), of[ks], dpt);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = exp2f(st[r] * sl2 - lse2);
        if (!full) {
          const int j = j0 + kh * 32 + mfma32_row(r, lane);
          if (!(visible(qi, j, W) && j < S)) pv = 0.f;
        }
        ds[r] = pv * (dpt[r] - di);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16x8_t db = pack8(&ds[hf * 8]);
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
          const bf16_t* kr = Kt + (mb * 32 + (lane & 31)) * kTLD + kh * 32 + hf * 16;
          dq[mb] = mfma32(ld_frag_reordered(kr, lane), db, dq[mb]);
        }
      }
    }
  }
  if (qi < S) {
    bf16_t* row = dqkv + ((int64_t)b * S + qi) * ldd + h * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * (lane >> 5);
        uint2 u;
        u.x = pack_bf2(dq[mb][4 * g] * scale, dq[mb][4 * g + 1] * scale);
        u.y = pack_bf2(dq[mb][4 * g + 2] * scale, dq[mb][4 * g + 3] * scale);
        *reinterpret_cast<uint2*>(row + d0) = u;
      }
  }
}

// ------------------------------------------------------------------ fp32 SIMT
template <int D>
__global__ __launch_bounds__(128) void swa_fwd_simt(const float* __restrict__ qkv, int64_t ldq,
                                                    float* __restrict__ out, int64_t ldo,
                                                    float* __restrict__ lse, int B, int S, int H,
                                                    int W, float scale) {
  const int64_t idx = (int64_t)blockIdx.x * 128 + threadIdx.x;
  if (idx >= (int64_t)B * H * S) return;
  const int i = idx % S, h = (idx / S) % H, b = idx / ((int64_t)S * H);
  const int A = H * D;
  const float* base = qkv + (int64_t)b * S * ldq;
  float q[D], acc[D];
  for (int c = 0; c < D; ++c) { q[c] = base[(int64_t)i * ldq + h * D + c]; acc[c] = 0.f; }
  const int jlo = max(0, i - W + 1);
  float mx = -INFINITY;
  for (int j = jlo; j <= i; ++j) {
    const float* k = base + (int64_t)j * ldq + A + h * D;
    float s = 0.f;
    for (int c = 0; c < D; ++c) s += q[c] * k[c];
    mx = fmaxf(mx, s * scale);
  }
  float l = 0.f;
  for (int j = jlo; j <= i; ++j) {
    const float* k = base + (int64_t)j * ldq + A + h * D;
    const float* v = base + (int64_t)j * ldq + 2 * A + h * D;
    float s = 0.f;
    for (int c = 0; c < D; ++c) s += q[c] * k[c];
    const float p = expf(s * scale - mx);
    l += p;
    for (int c = 0; c < D; ++c) acc[c] += p * v[c];
  }
  float* orow = out + ((int64_t)b * S + i) * ldo + h * D;
  for (int c = 0; c < D; ++c) orow[c] = acc[c] / l;
  lse[idx] = mx + logf(l);
}

template <int D>
__global__ __launch_bounds__(128) void swa_bwd_dq_simt(const float* __restrict__ qkv, int64_t ldq,
                                                       const float* __restrict__ d_o, int64_t ld_do,
                                                       const float* __restrict__ lse,
                                                       const float* __restrict__ dvec,
                                                       float* __restrict__ dqkv, int64_t ldd,
                                                       int B, int S, int H, int W, float scale) {
  const int64_t idx = (int64_t)blockIdx.x * 128 + threadIdx.x;
  if (idx >= (int64_t)B * H * S) return;
  const int i = idx % S, h = (idx / S) % H, b = idx / ((int64_t)S * H);
  const int A = H * D;
  const float* base = qkv + (int64_t)b * S * ldq;
  float q[D], go[D], acc[D];
  for (int c = 0; c < D; ++c) {
    q[c] = base[(int64_t)i * ldq + h * D + c];
    go[c] = d_o[((int64_t)b * S + i) * ld_do + h * D + c];
    acc[c] = 0.f;
  }
  const float L = lse[idx], Di = dvec[idx];
  for (int j = max(0, i - W + 1); j <= i; ++j) {
    const float* k = base + (int64_t)j * ldq + A + h * D;
    const float* v = base + (int64_t)j * ldq + 2 * A + h * D;
    float s = 0.f, dp = 0.f;
    for (int c = 0; c < D; ++c) { s += q[c] * k[c]; dp += go[c] * v[c]; }
    const float ds = expf(s * scale - L) * (dp - Di);
    for (int c = 0; c < D; ++c) acc[c] += ds * k[c];
  }
  float* row = dqkv + ((int64_t)b * S + i) * ldd + h * D;
  for (int c = 0; c < D; ++c) row[c] = acc[c] * scale;
}

template <int D>
__global__ __launch_bounds__(128) void swa_bwd_dkdv_simt(
    const float* __restrict__ qkv, int64_t ldq, const float* __restrict__ d_o, int64_t ld_do,
    const float* __restrict__ lse, const float* __restrict__ dvec, float* __restrict__ dqkv,
    int64_t ldd, int B, int S, int H, int W, float scale) {
  const int64_t idx = (int64_t)blockIdx.x * 128 + threadIdx.x;
  if (idx >= (int64_t)B * H * S) return;
  const int j = idx % S, h = (idx / S) % H, b = idx / ((int64_t)S * H);
  const int A = H * D;
  const float* base = qkv + (int64_t)b * S * ldq;
  float k[D], v[D], dk[D], dv[D];
  for (int c = 0; c < D; ++c) {
    k[c] = base[(int64_t)j * ldq + A + h * D + c];
    v[c] = base[(int64_t)j * ldq + 2 * A + h * D + c];
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  const float* lse_b = lse + ((int64_t)b * H + h) * S;
  const float* dv_b = dvec + ((int64_t)b * H + h) * S;
  for (int i = j; i <= min(S - 1, j + W - 1); ++i) {
    const float* q = base + (int64_t)i * ldq + h * D;
    const float* go = d_o + ((int64_t)b * S + i) * ld_do + h * D;
    float s = 0.f, dp = 0.f;
    for (int c = 0; c < D; ++c) { s += q[c] * k[c]; dp += go[c] * v[c]; }
    const float p = expf(s * scale - lse_b[i]);
    const float ds = p * (dp - dv_b[i]);
    for (int c = 0; c < D; ++c) { dv[c] += p * go[c]; dk[c] += ds * q[c]; }
  }
  float* row = dqkv + ((int64_t)b * S + j) * ldd + h * D;
  for (int c = 0; c < D; ++c) { row[A + c] = dk[c] * scale; row[2 * A + c] = dv[c]; }
}

template <int D>
hipError_t fwd_d(int dtype, const SwaDesc& a, void* o, int64_t ldo, float* lse, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)D);
  if (dtype == 1) {
    dim3 grid((a.seq + kBQ - 1) / kBQ, a.n_heads, a.batch);
    const int64_t ldl = 2 * (int64_t)a.n_heads * D;
    if (a.qk_lo != nullptr)
      hipLaunchKernelGGL((swa_fwd_mfma<D, true>), grid, dim3(kSwaThreads), 0, s,
                         (const bf16_t*)a.qkv, a.ld_qkv, (const bf16_t*)a.qk_lo, ldl,
                         (bf16_t*)o, ldo, lse, a.seq, a.n_heads, a.window, scale * kLog2e);
    else
      hipLaunchKernelGGL((swa_fwd_mfma<D, false>), grid, dim3(kSwaThreads), 0, s,
                         (const bf16_t*)a.qkv, a.ld_qkv, (const bf16_t*)nullptr, ldl,
                         (bf16_t*)o, ldo, lse, a.seq, a.n_heads, a.window, scale * kLog2e);
  } else {
    const int64_t n = (int64_t)a.batch * a.n_heads * a.seq;
    hipLaunchKernelGGL((swa_fwd_simt<D>), dim3((n + 127) / 128), dim3(128), 0, s,
                       (const float*)a.qkv, a.ld_qkv, (float*)o, ldo, lse, a.batch, a.seq,
                       a.n_heads, a.window, scale);
  }
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(int dtype, const SwaDesc& a, const void* o, int64_t ldo, const void* d_o,
                 int64_t ld_do, const float* lse, float* dvec, void* dqkv, int64_t ldd,
                 hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)D);
  const int64_t n = (int64_t)a.batch * a.n_heads * a.seq;
  if (dtype == 1) {
    hipLaunchKernelGGL((swa_rowdot<bf16_t>), dim3((n + 255) / 256), dim3(256), 0, s,
                       (const bf16_t*)d_o, ld_do, (const bf16_t*)o, ldo, dvec, a.batch, a.seq,
                       a.n_heads, D);
    dim3 grid((a.seq + kBQ - 1) / kBQ, a.n_heads, a.batch);
    const int64_t ldl = 2 * (int64_t)a.n_heads * D;
    const bf16_t* lo = (const bf16_t*)a.qk_lo;
    if (lo != nullptr) {
      hipLaunchKernelGGL((swa_bwd_dkdv_mfma<D, true>), grid, dim3(kSwaThreads), 0, s,
                         (const bf16_t*)a.qkv, a.ld_qkv, lo, ldl, (const bf16_t*)d_o, ld_do, lse,
                         (const float*)dvec, (bf16_t*)dqkv, ldd, a.seq, a.n_heads, a.window,
                         scale * kLog2e, scale);
      hipLaunchKernelGGL((swa_bwd_dq_mfma<D, true>), grid, dim3(kSwaThreads), 0, s,
                         (const bf16_t*)a.qkv, a.ld_qkv, lo, ldl, (const bf16_t*)d_o, ld_do, lse,
                         (const float*)dvec, (bf16_t*)dqkv, ldd, a.seq, a.n_heads, a.window,
                         scale * kLog2e, scale);
    } else {
      hipLaunchKernelGGL((swa_bwd_dkdv_mfma<D, false>), grid, dim3(kSwaThreads), 0, s,
                         (const bf16_t*)a.qkv, a.ld_qkv, lo, ldl, (const bf16_t*)d_o, ld_do, lse,
                         (const float*)dvec, (bf16_t*)dqkv, ldd, a.seq, a.n_heads, a.window,
                         scale * kLog2e, scale);
      hipLaunchKernelGGL((swa_bwd_dq_mfma<D, false>), grid, dim3(kSwaThreads), 0, s,
                         (const bf16_t*)a.qkv, a.ld_qkv, lo, ldl, (const bf16_t*)d_o, ld_do, lse,
                         (const float*)dvec, (bf16_t*)dqkv, ldd, a.seq, a.n_heads, a.window,
                         scale * kLog2e, scale);
    }
  } else {
    hipLaunchKernelGGL((swa_rowdot<float>), dim3((n + 255) / 256), dim3(256), 0, s,
                       (const float*)d_o, ld_do, (const float*)o, ldo, dvec, a.batch, a.seq,
                       a.n_heads, D);
    hipLaunchKernelGGL((swa_bwd_dkdv_simt<D>), dim3((n + 127) / 128), dim3(128), 0, s,
                       (const float*)a.qkv, a.ld_qkv, (const float*)d_o, ld_do, lse,
                       (const float*)dvec, (float*)dqkv, ldd, a.batch, a.seq, a.n_heads,
                       a.window, scale);
    hipLaunchKernelGGL((swa_bwd_dq_simt<D>), dim3((n + 127) / 128), dim3(128), 0, s,
                       (const float*)a.qkv, a.ld_qkv, (const float*)d_o, ld_do, lse,
                       (const float*)dvec, (float*)dqkv, ldd, a.batch, a.seq, a.n_heads,
                       a.window, scale);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swa_fwd(int dtype, const SwaDesc& a, void* o, int64_t ldo, float* lse,
                          hipStream_t s) {
  switch (a.head_dim) {
    case 64: return fwd_d<64>(dtype, a, o, ldo, lse, s);
    case 96: return fwd_d<96>(dtype, a, o, ldo, lse, s);
    default: return fwd_d<128>(dtype, a, o, ldo, lse, s);
  }
}

hipError_t launch_swa_bwd(int dtype, const SwaDesc& a, const void* o, int64_t ldo,
                          const void* d_o, int64_t ld_do, const float* lse, float* dvec,
                          void* dqkv, int64_t ldd, hipStream_t s) {
  switch (a.head_dim) {
    case 64: return bwd_d<64>(dtype, a, o, ldo, d_o, ld_do, lse, dvec, dqkv, ldd, s);
    case 96: return bwd_d<96>(dtype, a, o, ldo, d_o, ld_do, lse, dvec, dqkv, ldd, s);
    default: return bwd_d<128>(dtype, a, o, ldo, d_o, ld_do, lse, dvec, dqkv, ldd, s);
  }
}

}  // namespace ptb
