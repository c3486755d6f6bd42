// Causal sliding-window attention (MegaScale study guide, ch.2 §2.2 technique
// table, SWA row: every token attends to a fixed window of w tokens, so the
// cost is O(s*w) instead of O(s*s)).  Key j is visible to query i of the same
// sequence iff 0 <= i - j < w; scores are scaled by 1/sqrt(d).
//
// bf16 path, 32x32 blocks with v_mfma_f32_32x32x16_bf16.  Forward and dQ:
// one workgroup = 8 waves over 128 queries; waves w and w + 4 own the same 32
// queries and take the first and second 32 keys of every 64-key tile, so two
// waves share each SIMD and overlap one's softmax with the other's MFMAs;
// their partial results are merged through LDS at the end.  dK/dV: one
// workgroup = 4 waves, each owning 32 keys.
//   * forward: a block of 128 queries walks only the 64-key tiles that
//     intersect its band; each wave skips key halves outside its own band and
//     masks only those that cross the band edges.  Scores are computed
//     transposed (S^T = K Q^T) so that each lane holds 16 scores of ONE
//     query: the online softmax (running max and sum, base-2 exponent) then
//     needs a single lane exchange, and the probabilities already sit in
//     the B-operand layout of O^T += V^T P^T (keys reordered inside the K=16
//     step, the same order used to read V^T from LDS).  The log-sum-exp of
//     each query is written for the backward.
//   * every key/query tile moves from memory straight into LDS (row-major,
//     LDS-bound buffer loads, double-buffered so the next tile loads while
//     the current one is multiplied); the transposed operands (V^T, dO^T,
//     Q^T, K^T) are read from those row-major tiles with the transposing
//     LDS read, so no transposed copy is ever staged.
//   * backward (FlashAttention-2 style, no atomics, deterministic): one
//     kernel per 128-query block forms D_i = dO_i . O_i for its queries
//     (and stores it) and accumulates dQ^T += K^T dS^T with the transposed
//     formulation of the forward; then one kernel per 128-key block
//     accumulates dK and dV over the query tiles of the band (S = Q K^T,
//     P = exp(S - lse), dP = dO V^T, dS = P (dP - D), dV^T += dO^T P,
//     dK^T += Q^T dS).
// fp32 path: one thread per query (or key) looping over its window; it serves
// the fp32 workload only.
#include "common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Forward: how far (base-2 exponent) a score may exceed the running
// reference max before O and l are rescaled.
constexpr float kSlack = 8.f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBQ = 128, kBKV = 64, kSwaThreads = 256, kSwaWideThreads = 512;

__device__ __forceinline__ bf16x8_t ld_frag(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}
__device__ __forceinline__ bf16x8_t pack8(const float* v) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]),
                                                  pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])));
}
__device__ __forceinline__ bool visible(int i, int j, int w) { return j <= i && i - j < w; }

// LDS row stride (elements) of a 64-row tile of D columns: D plus a pad
// chosen so that the fragment reads of consecutive rows fall on distinct
// banks, both the 16-byte row reads (8 rows at a time) and the transposing
// 8-byte reads (4 rows of 32 bytes at a time): the stride in 4-byte banks is
// 36, 52 and 72 for D = 64, 96 and 128.
template <int D>
constexpr int kTileLd = D + (D == 128 ? 16 : 8);

// One 64-row tile (rows r0 .. r0 + 63 of a token-major matrix, D columns)
// goes from memory straight into LDS with buffer loads that carry the LDS
// bit: one wave instruction writes 1 KB of LDS, lane L's 16 bytes at byte
// 16 L, so the row-major LDS tile (kTileLd<D> elements per row) is covered
// by NI = kTileLd<D> / 8 instructions; instruction n is issued by wave
// n % 4.  voff[k] is the byte offset, inside a tile, of this lane's piece
// of instruction wave + 4k (kOutOfRange for a pad slot, which then loads
// zeros); the tile's first row goes into the scalar offset, so whole tiles
// load without writing any vector register (a vector register that an
// outstanding LDS-bound load used as its address is not rewritten before
// the load completes, and per-tile address arithmetic would stall on it).
// RAGGED (the sequence is not a multiple of 64 rows): rows at or beyond
// `lim` are steered out of the buffer's range lane by lane.
template <int D>
struct DmaRows {
  static constexpr int CH = D / 8, SL = kTileLd<D> / 8;
  static constexpr int NI = SL;             // 1 KB instructions per tile
  static constexpr int NW = (NI + 3) / 4;   // per wave, at most
  // instructions of one tile issued by wave w
  static constexpr int count(int w) { return (NI - w + 3) / 4; }
  uint32_t voff[NW];
  int row[NW];
  __device__ __forceinline__ void init(int wave, int lane, int64_t ld) {
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const int s = (wave + 4 * k) * 64 + lane, r = s / SL, c = s - r * SL;
      row[k] = r;
      voff[k] = c < CH ? (uint32_t)(((int64_t)r * ld + c * 8) * 2) : kOutOfRange;
    }
  }
  // `ragged` is a compile-time constant at every call site (inlined).
  __device__ __forceinline__ void issue(bool ragged, __amdgpu_buffer_rsrc_t rs, bf16_t* tile,
                                        int wave, int r0, int lim, int64_t ld) const {
    const uint32_t so = (uint32_t)((int64_t)r0 * ld * 2);
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const int n = wave + 4 * k;
      if (n < NI) {  // uniform over the wave
        if (!ragged) {
          // (through a local: handing the member element straight to the
          // builtin made the host compilation drop the kernels' launch stubs)
          const uint32_t vo = voff[k];
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + n * 512), 16, vo, so,
                                                   0, 0);
        } else {
          const uint32_t o =
              voff[k] != kOutOfRange && r0 + row[k] < lim ? voff[k] + so : kOutOfRange;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + n * 512), 16, o, 0,
                                                   0, 0);
        }
      }
    }
  }
};

// K/V (or Q/dO) tiles in flight: three stages where they fit in LDS next to
// each other (d <= 96), else two.  With three, the loads of tile t+2 are
// issued while tile t is multiplied and tile t+1 may still be landing.
template <int D>
constexpr int kSwaStages = D <= 96 ? 3 : 2;

// Waits until this wave has at most VM loads outstanding (the LDS-bound ones
// included) and no LDS reads, then joins the workgroup barrier.  VM0 is
// wave 0's allowance, VM1 that of waves 1-3 (wave 0 may issue more), VM4
// that of waves 4 and up (in the eight-wave kernels they issue no tile
// loads).
template <int VM0, int VM1, int VM4 = VM1>
__device__ __forceinline__ void tile_barrier(int wave) {
  static_assert(VM0 < 64 && VM1 < 64 && VM4 < 64, "vmcnt field");
  __builtin_amdgcn_sched_barrier(0);
  if (wave == 0)
    __builtin_amdgcn_s_waitcnt((VM0 & 15) | ((VM0 >> 4) << 14) | (7 << 4));
  else if (wave < 4)
    __builtin_amdgcn_s_waitcnt((VM1 & 15) | ((VM1 >> 4) << 14) | (7 << 4));
  else
    __builtin_amdgcn_s_waitcnt((VM4 & 15) | ((VM4 >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// The buffer covering one sequence's rows of a D-column block: rows 0 ..
// seq - 1 of a token-major matrix with leading dimension ld (the entry
// points keep every token-major matrix below 2^31 bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const bf16_t* p, int64_t ld, int seq,
                                                            int D) {
  return make_rsrc(p, (uint32_t)(((int64_t)(seq - 1) * ld + D) * 2));
}

// A-operand fragment of a transposed tile, read from the row-major LDS tile
// (row stride LD) with ds_read_b64_tr_b16: M = 32 columns (dbase ..), K = 16
// tile rows from row0 taken in the order of probabilities held in MFMA
// output layout (MFMA K index 0-3 -> rows 0-3, 4-7 -> 8-11, 8-11 -> 4-7,
// 12-15 -> 12-15).  In each group of 16 lanes, lane i receives element i%4
// of the 4-value pieces addressed by lanes 4e + i/4 (e = 0..3), so lane j
// addresses tile row 4 (g/2) + j/4 at column 16 (g%2) + 4 (j%4); the second
// read covers the rows 8 further down.
template <int LD>
__device__ __forceinline__ bf16x8_t ld_frag_tr(const bf16_t* tile, int row0, int dbase, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int idx = (row0 + 4 * (g >> 1) + (j >> 2)) * LD + dbase + 16 * (g & 1) + 4 * (j & 3);
  const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)&tile[idx]);
  const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)&tile[idx + 8 * LD]);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}


// Workgroup -> (row block, head, sequence) of a launch over every row block
// of every head.  The hardware deals workgroups round-robin to the 8 XCDs;
// the remap gives each XCD a contiguous range of (sequence, head, block), so
// the row blocks of one head run on one XCD and share that head's K/V (or
// Q/dO) tiles in its L2 instead of fetching them once per XCD.
struct SwaBlock {
  int blk, h, b;
};
__device__ __forceinline__ SwaBlock swa_block(int S, int H) {
  const int total = gridDim.x, nb = (S + kBQ - 1) / kBQ, per = total >> 3;
  int l = blockIdx.x;
  if (l < (per << 3)) l = (l & 7) * per + (l >> 3);
  return {l % nb, (l / nb) % H, l / (nb * H)};
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
//
// Eight waves: waves w and w + 4 own the same 32 queries and split every
// 64-key tile, wave w taking keys 0-31 and wave w + 4 keys 32-63, each with
// its own running max, sum and output.  Two waves per SIMD then overlap one
// wave's softmax with the other's MFMAs, with the same LDS tiles as four
// waves would use.  At the end the partner wave hands its (max, sum, O) to
// wave w through LDS and wave w merges them, exactly as online softmax
// merges two blocks of keys.  K, K_lo and V tiles are staged in LDS (three
// stages for d <= 96, else two); waves 0-3 issue the loads, all eight meet
// at one barrier per tile.
template <int D, bool SPLIT, bool RAGGED>
__global__ __launch_bounds__(kSwaWideThreads) void swa_fwd_mfma(const bf16_t* __restrict__ qkv,
                                                                int64_t ldq,
                                                                const bf16_t* __restrict__ qk_lo,
                                                                int64_t ldl,
                                                                bf16_t* __restrict__ out,
                                                                int64_t ldo,
                                                                float* __restrict__ lse, int S,
                                                                int H, int W, float sl2) {
  constexpr int NS = kSwaStages<D>;
  constexpr int KLD = kTileLd<D>, TE = kBKV * KLD, TL = SPLIT ? TE : 8, T3 = NS > 2 ? TE : 8,
                TL3 = NS > 2 ? TL : 8;
  __shared__ __attribute__((aligned(16))) bf16_t K0[TE], K1[TE], K2[T3], V0[TE], V1[TE], V2[T3];
  __shared__ __attribute__((aligned(16))) bf16_t L0[TL], L1[TL], L2[TL3];
  const SwaBlock sb = swa_block(S, H);
  const int h = sb.h, b = sb.b;
  const int A = H * D;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int qgrp = wave & 3, half = wave >> 2;  // query group, key half of every tile
  const int q0 = sb.blk * kBQ;
  const int qw = q0 + qgrp * 32;
  const int qi = qw + (lane & 31);
  const bf16_t* base = qkv + (int64_t)b * S * ldq;
  const bf16_t* Qp = base + h * D;
  const bf16_t* Kp = base + A + h * D;
  const bf16_t* Vp = base + 2 * A + h * D;
  const bf16_t* lo_base = SPLIT ? qk_lo + (int64_t)b * S * ldl : nullptr;
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(Kp, ldq, S, D), rv = rows_rsrc(Vp, ldq, S, D);
  const __amdgpu_buffer_rsrc_t rl =
      SPLIT ? rows_rsrc(lo_base + A + h * D, ldl, S, D) : rk;
  const bool loader = wave < 4;
  DmaRows<D> dq_, dl_;
  dq_.init(qgrp, lane, ldq);
  if (SPLIT) dl_.init(qgrp, lane, ldl);
  // loads per tile of wave 0 and of waves 1-3 (the same for waves 1-3
  // whenever three stages are used); waves 4-7 issue none
  constexpr int NA = SPLIT ? 3 : 2;
  constexpr int C0 = NA * DmaRows<D>::count(0), C1 = NA * DmaRows<D>::count(1);
  static_assert(NS == 2 || (DmaRows<D>::count(1) == DmaRows<D>::count(3)), "load counts");

  const int qlast = min(q0 + kBQ, S) - 1;
  const int kt_lo = max(0, q0 - W + 1) / kBKV, kt_hi = qlast / kBKV;
  // tiles past kt_hi reload tile kt_hi: they are never used, but every body
  // issues the same loads, so the load counts the waits assume hold
  auto issue = [&](bf16_t* k, bf16_t* kl, bf16_t* v, int kt) {
    if (!loader) return;
    const int r0 = min(kt, kt_hi) * kBKV;
    dq_.issue(RAGGED, rk, k, wave, r0, S, ldq);
    if (SPLIT) dl_.issue(RAGGED, rl, kl, wave, r0, S, ldl);
    dq_.issue(RAGGED, rv, v, wave, r0, S, ldq);
  };

  bf16x8_t qf[D / 16], qf_lo[D / 16];
  load_row_frags<D>(qf, Qp, ldq, qi, S, lane);
  if (SPLIT) load_row_frags<D>(qf_lo, lo_base + h * D, ldl, qi, S, lane);
  issue(K0, L0, V0, kt_lo);
  if (NS > 2) issue(K1, L1, V1, kt_lo + 1);
  f32x16_t o[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const bool wave_live = qw < S;

  // tile kt is in (Ks, Ks_lo, Vs); tile kt + NS - 1 goes into (nk, nl, nv),
  // the stage tile kt - 1 used
  auto body = [&](const bf16_t* Ks, const bf16_t* Ks_lo, const bf16_t* Vs, bf16_t* nk,
                  bf16_t* nl, bf16_t* nv, int kt) {
    tile_barrier<(NS - 2) * C0, (NS - 2) * C1, 0>(wave);
    issue(nk, nl, nv, kt + NS - 1);
    const int j0 = kt * kBKV + half * 32;  // this wave's 32 keys
    if (kt > kt_hi || !wave_live || j0 > qw + 31 || j0 + 31 < qw - W + 1) return;
    const bool full = (j0 + 31 <= qw) && (qw + 31 - j0 < W) && (j0 + 32 <= S);
    // two independent accumulation chains (even and odd K steps)
    f32x16_t st, st2;
#pragma unroll
    for (int r = 0; r < 16; ++r) { st[r] = 0.f; st2[r] = 0.f; }
    const int fo = (half * 32 + (lane & 31)) * KLD + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      f32x16_t& acc = (ks & 1) ? st2 : st;
      const bf16x8_t kf = ld_frag(Ks + fo + ks * 16);
      acc = mfma32(kf, qf[ks], acc);
      if (SPLIT) {
        acc = mfma32(kf, qf_lo[ks], acc);
        acc = mfma32(ld_frag(Ks_lo + fo + ks * 16), qf[ks], acc);
      }
    }
    float mblk = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float sv = (st[r] + st2[r]) * sl2;
      if (!full) {
        const int j = j0 + mfma32_row(r, lane);
        if (!(visible(qi, j, W) && j < S)) sv = -INFINITY;
      }
      st[r] = sv;
      mblk = fmaxf(mblk, sv);
    }
    mblk = fmaxf(mblk, __shfl_xor(mblk, 32, 64));
    // The reference max moves only when a score exceeds it by more than
    // 2^kSlack (or on the first visible key), so the rescale of O and l is
    // skipped for most tiles; probabilities then stay below 2^kSlack, and
    // the final normalisation uses the same reference, so the result is
    // the same up to rounding.
    const bool grow = mblk > m_run + kSlack;
    if (__any(grow)) {
      const float m_next = grow ? mblk : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_next);
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
      m_run = m_next;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(st[r] - m_use);
      l_run += p[r];
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bf16x8_t pb = pack8(&p[hf * 8]);
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
        o[mb] = mfma32(ld_frag_tr<KLD>(Vs, half * 32 + hf * 16, mb * 32, lane), pb, o[mb]);
    }
  };
  if constexpr (NS == 2) {
    for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
      body(K0, L0, V0, K1, L1, V1, kt);
      body(K1, L1, V1, K0, L0, V0, kt + 1);
    }
  } else {
    for (int kt = kt_lo; kt <= kt_hi; kt += 3) {
      body(K0, L0, V0, K2, L2, V2, kt);
      body(K1, L1, V1, K0, L0, V0, kt + 1);
      body(K2, L2, V2, K1, L1, V1, kt + 2);
    }
  }
  // every load has landed and every wave is done with the tiles: the tile
  // buffers now carry the second key half's partials to its partner wave
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* xch = reinterpret_cast<float*>(qgrp == 0 ? K0 : qgrp == 1 ? K1 : qgrp == 2 ? V0 : V1);
  static_assert((2 + 16 * (D / 32)) * 64 * 4 <= TE * 2, "exchange fits a tile buffer");
  if (half == 1) {
    xch[lane] = m_run;
    xch[64 + lane] = l_run;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[(2 + 16 * mb + r) * 64 + lane] = o[mb][r];
  }
  __syncthreads();
  if (half == 1) return;
  {
    const float mb_ = xch[lane], lb = xch[64 + lane];
    const float m = fmaxf(m_run, mb_);
    const float m_use = m == -INFINITY ? 0.f : m;
    const float fa = __builtin_amdgcn_exp2f(m_run - m_use), fb = __builtin_amdgcn_exp2f(mb_ - m_use);
    l_run = l_run * fa + lb * fb;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[mb][r] = o[mb][r] * fa + xch[(2 + 16 * mb + r) * 64 + lane] * fb;
    m_run = m;
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
// fp32 path (the bf16 path forms D inside the dQ kernel): one thread per
// (batch, head, query); the head's D values of dO and O move as 8-element
// vectors (D is a multiple of 8).
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
// Q, Q_lo and dO tiles double-buffered in LDS as in the forward; the
// log-sum-exp and D values of the next query tile ride in registers of the
// first wave and are written to LDS just before the barrier that publishes
// their tile.
template <int D, bool SPLIT, bool RAGGED>
__global__ __launch_bounds__(kSwaThreads) void swa_bwd_dkdv_mfma(
    const bf16_t* __restrict__ qkv, int64_t ldq, const bf16_t* __restrict__ qk_lo, int64_t ldl,
    const bf16_t* __restrict__ d_o, int64_t ld_do,
    const float* __restrict__ lse, const float* __restrict__ dvec, bf16_t* __restrict__ dqkv,
    int64_t ldd, int S, int H, int W, float sl2, float scale) {
  constexpr int NS = kSwaStages<D>;
  constexpr int KLD = kTileLd<D>, TE = kBKV * KLD, TL = SPLIT ? TE : 8, T3 = NS > 2 ? TE : 8,
                TL3 = NS > 2 ? TL : 8;
  __shared__ __attribute__((aligned(16))) bf16_t Q0[TE], Q1[TE], Q2[T3], O0[TE], O1[TE], O2[T3];
  __shared__ __attribute__((aligned(16))) bf16_t L0[TL], L1[TL], L2[TL3];
  __shared__ __attribute__((aligned(16))) float ls0[kBKV], ls1[kBKV], ls2[kBKV];
  __shared__ __attribute__((aligned(16))) float dd0[kBKV], dd1[kBKV], dd2[kBKV];
  const SwaBlock sb = swa_block(S, H);
  const int h = sb.h, b = sb.b;
  const int A = H * D;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int k0 = sb.blk * kBQ;
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
  const __amdgpu_buffer_rsrc_t rq = rows_rsrc(Qp, ldq, S, D), ro = rows_rsrc(dOp, ld_do, S, D);
  const __amdgpu_buffer_rsrc_t rl = SPLIT ? rows_rsrc(lo_base + h * D, ldl, S, D) : rq;
  // the tile's log-sum-exp and D values (64 floats each) go to LDS with one
  // 4-byte LDS-bound load per lane, issued by wave 0
  const __amdgpu_buffer_rsrc_t rls = make_rsrc(lse_b, (uint32_t)S * 4u);
  const __amdgpu_buffer_rsrc_t rdd = make_rsrc(dv_b, (uint32_t)S * 4u);
  uint32_t lane4 = (uint32_t)lane * 4u;
  asm volatile("" : "+v"(lane4));  // kept in one register, not recomputed per load
  DmaRows<D> dq_, dl_, do_;
  dq_.init(wave, lane, ldq);
  if (SPLIT) dl_.init(wave, lane, ldl);
  do_.init(wave, lane, ld_do);
  constexpr int NA = SPLIT ? 3 : 2;
  constexpr int C0 = NA * DmaRows<D>::count(0) + 2, C1 = NA * DmaRows<D>::count(1);
  static_assert(NS == 2 || (DmaRows<D>::count(1) == DmaRows<D>::count(3)), "load counts");

  const int klast = min(k0 + kBQ, S) - 1;
  const int qt_lo = k0 / kBKV, qt_hi = min(S - 1, klast + W - 1) / kBKV;
  // tiles past qt_hi reload tile qt_hi (never used; keeps the load counts)
  auto issue = [&](bf16_t* q, bf16_t* ql, bf16_t* o, float* ls, float* dd, int qt) {
    const int i0 = min(qt, qt_hi) * kBKV;
    dq_.issue(RAGGED, rq, q, wave, i0, S, ldq);
    if (SPLIT) dl_.issue(RAGGED, rl, ql, wave, i0, S, ldl);
    do_.issue(RAGGED, ro, o, wave, i0, S, ld_do);
    if (wave == 0) {
      // whole tiles: fixed lane offset plus the tile's scalar offset; the
      // ragged variant folds the tile offset into the lane offset and sends
      // rows at or beyond S out of range
      const uint32_t so = (uint32_t)i0 * 4u;
      const uint32_t vo = !RAGGED ? lane4 : (i0 + lane < S ? lane4 + so : kOutOfRange);
      const uint32_t sv = RAGGED ? 0u : so;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rls, (lds_void_t*)ls, 4, vo, sv, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rdd, (lds_void_t*)dd, 4, vo, sv, 0, 0);
    }
  };

  bf16x8_t kf[D / 16], vf[D / 16], kf_lo[D / 16];
  load_row_frags<D>(kf, Kp, ldq, kj, S, lane);
  load_row_frags<D>(vf, Vp, ldq, kj, S, lane);
  if (SPLIT) load_row_frags<D>(kf_lo, lo_base + A + h * D, ldl, kj, S, lane);
  issue(Q0, L0, O0, ls0, dd0, qt_lo);
  if (NS > 2) issue(Q1, L1, O1, ls1, dd1, qt_lo + 1);
  f32x16_t dk[D / 32], dv[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[mb][r] = 0.f; dv[mb][r] = 0.f; }
  const bool wave_live = kw < S;

  // tile qt is in (Qs, Qs_lo, dOs, lse_s, dv_s); tile qt + NS - 1 goes into
  // the n* arrays, the stage tile qt - 1 used
  auto body = [&](const bf16_t* Qs, const bf16_t* Qs_lo, const bf16_t* dOs, const float* lse_s,
                  const float* dv_s, bf16_t* nq, bf16_t* nql, bf16_t* no, float* nls, float* ndd,
                  int qt) {
    tile_barrier<(NS - 2) * C0, (NS - 2) * C1>(wave);
    issue(nq, nql, no, nls, ndd, qt + NS - 1);
    const int i0 = qt * kBKV;
    if (qt > qt_hi || !wave_live || i0 > kw + 31 + W - 1 || i0 + kBKV - 1 < kw) return;
    const bool full = (i0 >= kw + 31) && (i0 + kBKV - 1 - kw < W) && (i0 + kBKV <= S);
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      // scores in two accumulation chains (even and odd K steps), dP in a third
      f32x16_t s, s2, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) { s[r] = 0.f; s2[r] = 0.f; dp[r] = 0.f; }
      const int fo = (qh * 32 + (lane & 31)) * KLD + (lane >> 5) * 8;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        f32x16_t& acc = (ks & 1) ? s2 : s;
        const bf16x8_t qa = ld_frag(Qs + fo + ks * 16);
        acc = mfma32(qa, kf[ks], acc);
        if (SPLIT) {
          acc = mfma32(qa, kf_lo[ks], acc);
          acc = mfma32(ld_frag(Qs_lo + fo + ks * 16), kf[ks], acc);
        }
        dp = mfma32(ld_frag(dOs + fo + ks * 16), vf[ks], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] += s2[r];
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
          float pv = __builtin_amdgcn_exp2f(s[r] * sl2 - lv[e] * kLog2e);
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
          dv[mb] = mfma32(ld_frag_tr<KLD>(dOs, qh * 32 + hf * 16, mb * 32, lane), pb, dv[mb]);
          dk[mb] = mfma32(ld_frag_tr<KLD>(Qs, qh * 32 + hf * 16, mb * 32, lane), db, dk[mb]);
        }
      }
    }
  };
  if constexpr (NS == 2) {
    for (int qt = qt_lo; qt <= qt_hi; qt += 2) {
      body(Q0, L0, O0, ls0, dd0, Q1, L1, O1, ls1, dd1, qt);
      body(Q1, L1, O1, ls1, dd1, Q0, L0, O0, ls0, dd0, qt + 1);
    }
  } else {
    for (int qt = qt_lo; qt <= qt_hi; qt += 3) {
      body(Q0, L0, O0, ls0, dd0, Q2, L2, O2, ls2, dd2, qt);
      body(Q1, L1, O1, ls1, dd1, Q0, L0, O0, ls0, dd0, qt + 1);
      body(Q2, L2, O2, ls2, dd2, Q1, L1, O1, ls1, dd1, qt + 2);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may still be writing LDS when the workgroup ends
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
// Eight waves, split like the forward: waves w and w + 4 own the same 32
// queries and take keys 0-31 and 32-63 of every K/V tile; the partner's dQ
// partial is added through LDS at the end.  K, K_lo and V tiles are staged
// in LDS as in the forward.
template <int D, bool SPLIT, bool RAGGED>
__global__ __launch_bounds__(kSwaWideThreads) void swa_bwd_dq_mfma(
    const bf16_t* __restrict__ qkv, int64_t ldq, const bf16_t* __restrict__ qk_lo, int64_t ldl,
    const bf16_t* __restrict__ d_o, int64_t ld_do, const bf16_t* __restrict__ o, int64_t ldo,
    const float* __restrict__ lse, float* __restrict__ dvec, bf16_t* __restrict__ dqkv,
    int64_t ldd, int S, int H, int W, float sl2, float scale) {
  constexpr int NS = kSwaStages<D>;
  constexpr int KLD = kTileLd<D>, TE = kBKV * KLD, TL = SPLIT ? TE : 8, T3 = NS > 2 ? TE : 8,
                TL3 = NS > 2 ? TL : 8;
  __shared__ __attribute__((aligned(16))) bf16_t K0[TE], K1[TE], K2[T3], V0[TE], V1[TE], V2[T3];
  __shared__ __attribute__((aligned(16))) bf16_t L0[TL], L1[TL], L2[TL3];
  const SwaBlock sb = swa_block(S, H);
  const int h = sb.h, b = sb.b;
  const int A = H * D;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int qgrp = wave & 3, half = wave >> 2;
  const int q0 = sb.blk * kBQ;
  const int qw = q0 + qgrp * 32;
  const int qi = qw + (lane & 31);
  const bf16_t* base = qkv + (int64_t)b * S * ldq;
  const bf16_t* Qp = base + h * D;
  const bf16_t* Kp = base + A + h * D;
  const bf16_t* Vp = base + 2 * A + h * D;
  const bf16_t* dOp = d_o + (int64_t)b * S * ld_do + h * D;
  const bf16_t* lo_base = SPLIT ? qk_lo + (int64_t)b * S * ldl : nullptr;
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(Kp, ldq, S, D), rv = rows_rsrc(Vp, ldq, S, D);
  const __amdgpu_buffer_rsrc_t rl =
      SPLIT ? rows_rsrc(lo_base + A + h * D, ldl, S, D) : rk;
  const bool loader = wave < 4;
  DmaRows<D> dq_, dl_;
  dq_.init(qgrp, lane, ldq);
  if (SPLIT) dl_.init(qgrp, lane, ldl);
  // loads per tile of wave 0 and of waves 1-3 (the same for waves 1-3
  // whenever three stages are used); waves 4-7 issue none
  constexpr int NA = SPLIT ? 3 : 2;
  constexpr int C0 = NA * DmaRows<D>::count(0), C1 = NA * DmaRows<D>::count(1);
  static_assert(NS == 2 || (DmaRows<D>::count(1) == DmaRows<D>::count(3)), "load counts");

  const int qlast = min(q0 + kBQ, S) - 1;
  const int kt_lo = max(0, q0 - W + 1) / kBKV, kt_hi = qlast / kBKV;
  // tiles past kt_hi reload tile kt_hi: they are never used, but every body
  // issues the same loads, so the load counts the waits assume hold
  auto issue = [&](bf16_t* k, bf16_t* kl, bf16_t* v, int kt) {
    if (!loader) return;
    const int r0 = min(kt, kt_hi) * kBKV;
    dq_.issue(RAGGED, rk, k, wave, r0, S, ldq);
    if (SPLIT) dl_.issue(RAGGED, rl, kl, wave, r0, S, ldl);
    dq_.issue(RAGGED, rv, v, wave, r0, S, ldq);
  };

  bf16x8_t qf[D / 16], of[D / 16], qf_lo[D / 16];
  load_row_frags<D>(qf, Qp, ldq, qi, S, lane);
  load_row_frags<D>(of, dOp, ld_do, qi, S, lane);
  if (SPLIT) load_row_frags<D>(qf_lo, lo_base + h * D, ldl, qi, S, lane);
  // D_i = dO_i . O_i for this wave's queries: lanes l and l + 32 hold the
  // two halves of each K=16 step of query l's row; the dK/dV kernel, launched
  // after this one, reads the values back (the first key half stores them)
  float di;
  {
    bf16x8_t ofo[D / 16];
    load_row_frags<D>(ofo, o + (int64_t)b * S * ldo + h * D, ldo, qi, S, lane);
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) part += bf2f(of[ks][e]) * bf2f(ofo[ks][e]);
    di = part + __shfl_xor(part, 32, 64);
    if (half == 0 && lane < 32 && qi < S) dvec[((int64_t)b * H + h) * S + qi] = di;
  }
  issue(K0, L0, V0, kt_lo);
  if (NS > 2) issue(K1, L1, V1, kt_lo + 1);
  const float lse2 = qi < S ? lse[((int64_t)b * H + h) * S + qi] * kLog2e : 0.f;
  f32x16_t dq[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[mb][r] = 0.f;
  const bool wave_live = qw < S;

  auto body = [&](const bf16_t* Ks, const bf16_t* Ks_lo, const bf16_t* Vs, bf16_t* nk,
                  bf16_t* nl, bf16_t* nv, int kt) {
    tile_barrier<(NS - 2) * C0, (NS - 2) * C1, 0>(wave);
    issue(nk, nl, nv, kt + NS - 1);
    const int j0 = kt * kBKV + half * 32;  // this wave's 32 keys
    if (kt > kt_hi || !wave_live || j0 > qw + 31 || j0 + 31 < qw - W + 1) return;
    const bool full = (j0 + 31 <= qw) && (qw + 31 - j0 < W) && (j0 + 32 <= S);
    // scores in two accumulation chains (even and odd K steps), dP in a third
    f32x16_t st, st2, dpt;
#pragma unroll
    for (int r = 0; r < 16; ++r) { st[r] = 0.f; st2[r] = 0.f; dpt[r] = 0.f; }
    const int fo = (half * 32 + (lane & 31)) * KLD + (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      f32x16_t& acc = (ks & 1) ? st2 : st;
      const bf16x8_t ka = ld_frag(Ks + fo + ks * 16);
      acc = mfma32(ka, qf[ks], acc);
      if (SPLIT) {
        acc = mfma32(ka, qf_lo[ks], acc);
        acc = mfma32(ld_frag(Ks_lo + fo + ks * 16), qf[ks], acc);
      }
      dpt = mfma32(ld_frag(Vs + fo + ks * 16), of[ks], dpt);
    }
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pv = __builtin_amdgcn_exp2f((st[r] + st2[r]) * sl2 - lse2);
      if (!full) {
        const int j = j0 + mfma32_row(r, lane);
        if (!(visible(qi, j, W) && j < S)) pv = 0.f;
      }
      ds[r] = pv * (dpt[r] - di);
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bf16x8_t db = pack8(&ds[hf * 8]);
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
        dq[mb] = mfma32(ld_frag_tr<KLD>(Ks, half * 32 + hf * 16, mb * 32, lane), db, dq[mb]);
    }
  };
  if constexpr (NS == 2) {
    for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
      body(K0, L0, V0, K1, L1, V1, kt);
      body(K1, L1, V1, K0, L0, V0, kt + 1);
    }
  } else {
    for (int kt = kt_lo; kt <= kt_hi; kt += 3) {
      body(K0, L0, V0, K2, L2, V2, kt);
      body(K1, L1, V1, K0, L0, V0, kt + 1);
      body(K2, L2, V2, K1, L1, V1, kt + 2);
    }
  }
  // every load has landed and every wave is done with the tiles: the tile
  // buffers now carry the second key half's dQ partial to its partner wave
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* xch = reinterpret_cast<float*>(qgrp == 0 ? K0 : qgrp == 1 ? K1 : qgrp == 2 ? V0 : V1);
  static_assert(16 * (D / 32) * 64 * 4 <= TE * 2, "exchange fits a tile buffer");
  if (half == 1) {
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[(16 * mb + r) * 64 + lane] = dq[mb][r];
  }
  __syncthreads();
  if (half == 1) return;
  if (qi < S) {
    bf16_t* row = dqkv + ((int64_t)b * S + qi) * ldd + h * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * (lane >> 5);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (dq[mb][4 * g + e] + xch[(16 * mb + 4 * g + e) * 64 + lane]) * scale;
        uint2 u;
        u.x = pack_bf2(v[0], v[1]);
        u.y = pack_bf2(v[2], v[3]);
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

template <int D, bool SP, bool RG>
void launch_fwd_mfma(const SwaDesc& a, void* o, int64_t ldo, float* lse, float scale,
                     hipStream_t s) {
  dim3 grid((a.seq + kBQ - 1) / kBQ * a.n_heads * a.batch);
  const int64_t ldl = 2 * (int64_t)a.n_heads * D;
  hipLaunchKernelGGL((swa_fwd_mfma<D, SP, RG>), grid, dim3(kSwaWideThreads), 0, s,
                     (const bf16_t*)a.qkv, a.ld_qkv, (const bf16_t*)a.qk_lo, ldl, (bf16_t*)o, ldo,
                     lse, a.seq, a.n_heads, a.window, scale * kLog2e);
}

// dQ first: it also writes D = rowsum(dO * O), which dK/dV then reads.
template <int D, bool SP, bool RG>
void launch_bwd_mfma(const SwaDesc& a, const void* o, int64_t ldo, const void* d_o,
                     int64_t ld_do, const float* lse, float* dvec, void* dqkv, int64_t ldd,
                     float scale, hipStream_t s) {
  dim3 grid((a.seq + kBQ - 1) / kBQ * a.n_heads * a.batch);
  const int64_t ldl = 2 * (int64_t)a.n_heads * D;
  const bf16_t* lo = (const bf16_t*)a.qk_lo;
  hipLaunchKernelGGL((swa_bwd_dq_mfma<D, SP, RG>), grid, dim3(kSwaWideThreads), 0, s,
                     (const bf16_t*)a.qkv, a.ld_qkv, lo, ldl, (const bf16_t*)d_o, ld_do,
                     (const bf16_t*)o, ldo, lse, dvec, (bf16_t*)dqkv, ldd, a.seq, a.n_heads,
                     a.window, scale * kLog2e, scale);
  hipLaunchKernelGGL((swa_bwd_dkdv_mfma<D, SP, RG>), grid, dim3(kSwaThreads), 0, s,
                     (const bf16_t*)a.qkv, a.ld_qkv, lo, ldl, (const bf16_t*)d_o, ld_do, lse,
                     (const float*)dvec, (bf16_t*)dqkv, ldd, a.seq, a.n_heads, a.window,
                     scale * kLog2e, scale);
}

template <int D>
hipError_t fwd_d(int dtype, const SwaDesc& a, void* o, int64_t ldo, float* lse, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)D);
  if (dtype == 1) {
    const bool sp = a.qk_lo != nullptr, rg = a.seq % kBKV != 0;
    if (sp && rg) launch_fwd_mfma<D, true, true>(a, o, ldo, lse, scale, s);
    else if (sp) launch_fwd_mfma<D, true, false>(a, o, ldo, lse, scale, s);
    else if (rg) launch_fwd_mfma<D, false, true>(a, o, ldo, lse, scale, s);
    else launch_fwd_mfma<D, false, false>(a, o, ldo, lse, scale, s);
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
    const bool sp = a.qk_lo != nullptr, rg = a.seq % kBKV != 0;
    auto* f = sp ? (rg ? launch_bwd_mfma<D, true, true> : launch_bwd_mfma<D, true, false>)
                 : (rg ? launch_bwd_mfma<D, false, true> : launch_bwd_mfma<D, false, false>);
    f(a, o, ldo, d_o, ld_do, lse, dvec, dqkv, ldd, scale, s);
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
