// GEMM engine of the block: C[m, n] = sum_k A(m, k) B(n, k) with either
// operand K-contiguous or M/N-contiguous, and fused epilogues.
//
// The parallel block (MegaScale study guide, ch.2 §2.2 technique table, PTB
// row) feeds ONE LayerNorm output to both branches and sums both branch
// outputs, so the four projections of the two branches become two GEMMs:
//   forward : [q|k|v|f] = xn w_in^T           (epilogue: split + GeLU)
//             y = [O | GeLU(f)] w_out^T (+ x) (epilogue: residual)
//   backward: dcat = dy w_out                 (epilogue: split + GeLU')
//             dw_out = dy^T cat, dw_in = dz^T xn, dxn = dz w_in
//
// bf16 path (gfx950 MFMA): 256x256 output tile per workgroup of 4 waves, each
// wave a 128x128 sub-tile of 4x4 v_mfma_f32_32x32x16_bf16 blocks with fp32
// accumulators; K step 64; A and B tiles staged through LDS (row stride 72
// elements so the 16-byte fragment reads of 16 consecutive rows hit distinct
// banks), double-buffered, with the next tile's global loads in flight during
// the current tile's MFMAs.  An M/N-contiguous operand is loaded as 8x8
// blocks and transposed in registers before the LDS store, so the MFMA
// fragment reads are always K-contiguous.  Edges are masked by the buffer
// unit's range check (zero fill), so any M, N, K is accepted.
//
// Tile order: the hardware deals workgroups round-robin to the 8 XCDs; the
// block index is remapped so that each XCD gets a contiguous range of tiles,
// walked M-fastest within groups of 8 M-tiles, so tiles that share B columns
// run on the same XCD's L2.
//
// fp32 path: a plain LDS-tiled SIMT kernel (64x64 tile, 4x4 outputs per
// thread) with the same epilogues; it serves the fp32 workload.
#include "common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDS_LD = BK + 8;      // elements per LDS row
constexpr int kGemmThreads = 256;
constexpr int kGroupM = 8;

// --------------------------------------------------------------- epilogues
// Each epilogue takes one accumulator value (operator(), used by the fp32
// kernel) or 8 consecutive columns of one row (store8, used by the MFMA
// kernel after staging through LDS; col % 8 == 0, columns >= ncols dropped).
template <typename T>
__device__ __forceinline__ void put8(T* p, const float (&v)[8], int valid) {
  if (valid >= 8) {
    Vec8<T>::store(p, v);
  } else {
    for (int e = 0; e < valid; ++e) Elt<T>::st(p + e, v[e]);
  }
}
template <typename T>
__device__ __forceinline__ void get8(const T* p, float (&v)[8], int valid) {
  if (valid >= 8) {
    Vec8<T>::load(p, v);
  } else {
    for (int e = 0; e < 8; ++e) v[e] = e < valid ? Elt<T>::ld(p + e) : 0.f;
  }
}

template <typename T>
struct EpiStore {
  T* c;
  int64_t ldc;
  __device__ __forceinline__ void operator()(int row, int col, float v) const {
    Elt<T>::st(c + (int64_t)row * ldc + col, v);
  }
  __device__ __forceinline__ void store8(int row, int col, const float (&v)[8], int ncols) const {
    put8(c + (int64_t)row * ldc + col, v, ncols - col);
  }
};

// qk_lo (bf16 path; may be null): receives, for the q and k columns, the
// bf16 rounding residual v - bf16(v), so q and k are kept as hi + lo pairs.
template <typename T>
struct EpiInFwd {
  T* qkv;
  T* qk_lo;
  T* f;
  T* cat;
  int a3, attn, ffn;
  __device__ __forceinline__ void operator()(int row, int col, float v) const {
    if (col < a3) {
      Elt<T>::st(qkv + (int64_t)row * a3 + col, v);
    } else {
      const int c = col - a3;
      Elt<T>::st(f + (int64_t)row * ffn + c, v);
      Elt<T>::st(cat + (int64_t)row * (attn + ffn) + attn + c, gelu_f(v));
    }
  }
  // a3 and 2*attn are multiples of 8, so a chunk never straddles a border
  __device__ __forceinline__ void store8(int row, int col, const float (&v)[8], int ncols) const {
    const int valid = ncols - col;
    if (col < a3) {
      put8(qkv + (int64_t)row * a3 + col, v, valid);
      if (qk_lo != nullptr && col < 2 * attn) {
        float lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = v[e] - Elt<T>::ld_rounded(v[e]);
        put8(qk_lo + (int64_t)row * (2 * attn) + col, lo, valid);
      }
    } else {
      const int c = col - a3;
      put8(f + (int64_t)row * ffn + c, v, valid);
      float g[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = gelu_f(v[e]);
      put8(cat + (int64_t)row * (attn + ffn) + attn + c, g, valid);
    }
  }
};

template <typename T>
struct EpiOutFwd {
  T* y;
  const T* x;
  int64_t ld;
  int add;
  __device__ __forceinline__ void operator()(int row, int col, float v) const {
    const int64_t o = (int64_t)row * ld + col;
    if (add) v += Elt<T>::ld(x + o);
    Elt<T>::st(y + o, v);
  }
  __device__ __forceinline__ void store8(int row, int col, const float (&v)[8], int ncols) const {
    const int64_t o = (int64_t)row * ld + col;
    const int valid = ncols - col;
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = v[e];
    if (add) {
      float xv[8];
      get8(x + o, xv, valid);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] += xv[e];
    }
    put8(y + o, r, valid);
  }
};

template <typename T>
struct EpiDcat {
  const T* f;
  T* d_o;
  T* dz;
  int attn, ffn;
  __device__ __forceinline__ void operator()(int row, int col, float v) const {
    if (col < attn) {
      Elt<T>::st(d_o + (int64_t)row * attn + col, v);
    } else {
      const int c = col - attn;
      const float fv = Elt<T>::ld(f + (int64_t)row * ffn + c);
      Elt<T>::st(dz + (int64_t)row * (3 * attn + ffn) + 3 * attn + c, v * gelu_grad_f(fv));
    }
  }
  // attn is a multiple of 8, so a chunk never straddles the O / FC2 border
  __device__ __forceinline__ void store8(int row, int col, const float (&v)[8], int ncols) const {
    const int valid = ncols - col;
    if (col < attn) {
      put8(d_o + (int64_t)row * attn + col, v, valid);
    } else {
      const int c = col - attn;
      float fv[8], r[8];
      get8(f + (int64_t)row * ffn + c, fv, valid);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = v[e] * gelu_grad_f(fv[e]);
      put8(dz + (int64_t)row * (3 * attn + ffn) + 3 * attn + c, r, valid);
    }
  }
};

// --------------------------------------------------------------- tile order
constexpr int kMaxPerm = 128;

// Block -> output tile.  The hardware deals workgroups round-robin to the 8
// XCDs (block b runs on XCD b % 8); the remap gives each XCD a contiguous
// range of logical tiles, walked M-fastest within groups of kGroupM M-tiles,
// so tiles sharing a B panel run on the same XCD and its L2.  `perm`
// (optional) reorders the N tiles, e.g. to spread tiles with a longer K loop
// evenly over the XCD ranges.
__device__ __forceinline__ void tile_coords(int bid, int ntm, int ntn, const int16_t* perm,
                                            int& tm, int& tn) {
  const int ntiles = ntm * ntn;
  const int xcd = bid & 7, local = bid >> 3;
  const int full = ntiles >> 3, rem = ntiles & 7;
  const int logical = xcd < rem ? xcd * (full + 1) + local
                                : rem * (full + 1) + (xcd - rem) * full + local;
  const int per_group = kGroupM * ntn;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(ntm - first_m, kGroupM);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
  if (perm != nullptr) tn = perm[tn];
}

// --------------------------------------------------------------- bf16 loaders
// One 256 x 64 operand tile (256 rows of the M or N dimension, 64 of K).
template <int LAY>
struct TileLoader {
  uint4 r[8];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int row0, int rows, int k0,
                                       int K, int64_t ld) {
    const int t = threadIdx.x;
    if (LAY == kKContig) {
      const int c = t & 7, rr = t >> 3;
      const int k = k0 + c * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = row0 + rr + 32 * i;
        const uint32_t off = (row < rows && k < K)
                                 ? (uint32_t)(((int64_t)row * ld + k) * 2)
                                 : kOutOfRange;
        r[i] = buf_load16(rs, off);
      }
    } else {
      const int kb = t & 7, mb = t >> 3;
      const int row = row0 + mb * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = k0 + kb * 8 + i;
        const uint32_t off = (k < K && row < rows)
                                 ? (uint32_t)(((int64_t)k * ld + row) * 2)
                                 : kOutOfRange;
        r[i] = buf_load16(rs, off);
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds) const {
    const int t = threadIdx.x;
    if (LAY == kKContig) {
      const int c = t & 7, rr = t >> 3;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint4*>(lds + (rr + 32 * i) * LDS_LD + c * 8) = r[i];
    } else {
      const int kb = t & 7, mb = t >> 3;
      uint4 tr[8];
      transpose8x8(r, tr);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint4*>(lds + (mb * 8 + j) * LDS_LD + kb * 8) = tr[j];
    }
  }
};

// a2 (optional, same layout and leading dimension as a): output tiles whose
// first column lies below n_split accumulate a second K pass over a2 with
// the same B, i.e. C = (A + A2) B^T there.  The input projection uses it to
// form q and k from the LayerNorm output split into its bf16 value and bf16
// residual, so the attention scores do not inherit the rounding of xn.
struct GemmArgs {
  const bf16_t* a;
  const bf16_t* b;
  const bf16_t* a2;
  int M, N, K;
  int n_split;
  int64_t lda, ldb;
  uint32_t a_bytes, b_bytes;
  int use_perm;
  int16_t perm[kMaxPerm];  // N-tile order (when use_perm)
};

// Scheduling groups of one pipeline phase (masks: 0x008 MFMA, 0x020 memory
// read, 0x100 LDS read, 0x200 LDS write), each closed by a full scheduling
// barrier: interleave<M>: 8 x (1 MFMA, 1 op M) then the other 8 MFMAs;
// interleave3<M1, M2, M3>: 8 x (1 MFMA, 1 op M1), then 8 x (1 MFMA, 1 op M2,
// 1 op M3).
template <int M>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(M, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  __builtin_amdgcn_sched_barrier(0);
}
template <int M1, int M2, int M3>
__device__ __forceinline__ void interleave3() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(M1, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(M2, 1, 0);
    __builtin_amdgcn_sched_group_barrier(M3, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// 16 MFMAs of one K=16 step: the wave's 128x128 accumulators.
__device__ __forceinline__ void mma_step(f32x16_t (&acc)[4][4], const bf16x8_t (&fa)[4],
                                         const bf16x8_t (&fb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
}
// This lane's A and B fragments of K step ks from one LDS stage.
__device__ __forceinline__ void read_frags(bf16x8_t (&fa)[4], bf16x8_t (&fb)[4],
                                           const bf16_t* As, const bf16_t* Bs, int ks) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    fa[i] = *reinterpret_cast<const bf16x8_t*>(As + i * 32 * LDS_LD + ks * 16);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    fb[j] = *reinterpret_cast<const bf16x8_t*>(Bs + j * 32 * LDS_LD + ks * 16);
}

// Main loop as a three-stage pipeline over K tiles t = 0, 1, ... (tiles
// nk1.. of a two-pass tile read a2): while the MFMAs consume tile t from one
// LDS stage, tile t+1 (already in registers) is written to the other stage
// and tile t+2 is fetched from memory, split over the four K=16 steps so that
// LDS and memory instructions sit between MFMAs; the fragments of the next
// K=16 step are read from LDS one step ahead (two register sets).  Tiles at
// or beyond the end load out of range (zeros, no memory traffic), so the loop
// body has no branches.  One barrier per K tile.
template <int ALAY, int BLAY, class Epi>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_kernel(GemmArgs g, Epi epi) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[2][2][BM * LDS_LD];
  const int ntm = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, ntm, ntn, g.use_perm ? g.perm : nullptr, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, g.a_bytes);
  const __amdgpu_buffer_rsrc_t ra2 = make_rsrc(g.a2 != nullptr ? g.a2 : g.a, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.b, g.b_bytes);
  TileLoader<ALAY> la;
  TileLoader<BLAY> lb;
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk1 = (g.K + BK - 1) / BK;
  const int nk = (g.a2 != nullptr && n0 < g.n_split) ? 2 * nk1 : nk1;
  auto load_a = [&](int t) {
    const int kk = t < nk1 ? t : t - nk1;
    la.load(t < nk1 ? ra : ra2, m0, g.M, kk * BK, t < nk ? g.K : 0, g.lda);
  };
  auto load_b = [&](int t) {
    const int kk = t < nk1 ? t : t - nk1;
    lb.load(rb, n0, g.N, kk * BK, t < nk ? g.K : 0, g.ldb);
  };

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int frag_off = (lane & 31) * LDS_LD + (lane >> 5) * 8;
  const int a_off = wm * 128 * LDS_LD + frag_off, b_off = wn * 128 * LDS_LD + frag_off;

  load_a(0);
  load_b(0);
  la.store(lds[0][0]);
  lb.store(lds[0][1]);
  load_a(1);
  load_b(1);
  __syncthreads();
  bf16x8_t fa[2][4], fb[2][4];
  read_frags(fa[0], fb[0], lds[0][0] + a_off, lds[0][1] + b_off, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1, nxt = cur ^ 1;
    const bf16_t* As = lds[cur][0] + a_off;
    const bf16_t* Bs = lds[cur][1] + b_off;
    // Each phase: one K=16 MFMA group plus the memory work of the pipeline.
    // The group barriers interleave them (MFMA, memory op, MFMA, ...) so the
    // MFMAs, which only use fragments read in the previous phase, never wait
    // on this phase's LDS or memory traffic; sched_barrier(0) closes a phase.
    // Each operand's registers are refilled in the same phase that writes
    // them to LDS, which gives every memory load four phases of lead.
    read_frags(fa[1], fb[1], As, Bs, 1);
    la.store(lds[nxt][0]);
    load_a(kt + 2);
    mma_step(acc, fa[0], fb[0]);
    interleave3<0x100, 0x200, 0x020>();
    read_frags(fa[0], fb[0], As, Bs, 2);
    mma_step(acc, fa[1], fb[1]);
    interleave<0x100>();
    read_frags(fa[1], fb[1], As, Bs, 3);
    lb.store(lds[nxt][1]);
    load_b(kt + 2);
    mma_step(acc, fa[0], fb[0]);
    interleave3<0x100, 0x200, 0x020>();
    // Every wave has now written tile t+1 and read its last fragments of
    // tile t, so after this barrier the first fragments of tile t+1 can be
    // read while the last MFMA group of tile t runs from registers.
    __syncthreads();
    read_frags(fa[0], fb[0], lds[nxt][0] + a_off, lds[nxt][1] + b_off, 0);
    mma_step(acc, fa[1], fb[1]);
    interleave<0x100>();
  }
  __syncthreads();

  // Epilogue, one row of four 32x32 accumulator blocks at a time: each wave
  // stages its 32x128 strip in its own LDS area (fp32; block j at word
  // j*kStageBlk + {0,4,32,36}[j] so the row-chunk reads of the four blocks
  // fall on different banks) with a short fully unrolled loop, then re-reads
  // it as 8-column row chunks (4 rows x 128 columns per wave instruction) and
  // runs the epilogue in a rolled loop, so every lane issues 16-byte stores.
  constexpr int kStageRow = 36, kStageBlk = 1216;
  float* stage = reinterpret_cast<float*>(&lds[0][0][0]) + wave * (4 * kStageBlk);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float* blk = stage + j * kStageBlk + (j & 1) * 4 + (j >> 1) * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) blk[mfma32_row(r, lane) * kStageRow + (lane & 31)] = acc[i][j][r];
    }
    __syncthreads();
#pragma unroll 1
    for (int c = lane; c < 32 * 16; c += 64) {
      const int rr = c >> 4, jc = c & 15, j = jc >> 2, c8 = (jc & 3) * 8;
      const float* src = stage + j * kStageBlk + (j & 1) * 4 + (j >> 1) * 32 + rr * kStageRow + c8;
      const float4 lo = *reinterpret_cast<const float4*>(src);
      const float4 hi = *reinterpret_cast<const float4*>(src + 4);
      const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      const int row = m0 + wm * 128 + i * 32 + rr;
      const int col = n0 + wn * 128 + j * 32 + c8;
      if (row < g.M && col < g.N) epi.store8(row, col, v, g.N);
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------- fp32 SIMT
struct GemmArgsF32 {
  const float* a;
  const float* b;
  int M, N, K;
  int64_t lda, ldb;
};

template <int ALAY, int BLAY, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgsF32 g, Epi epi) {
  constexpr int T = 64, TK = 16;
  __shared__ float As[TK][T + 1], Bs[TK][T + 1];
  const int ntn = (g.N + T - 1) / T;
  const int m0 = (blockIdx.x / ntn) * T, n0 = (blockIdx.x % ntn) * T;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += TK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = threadIdx.x + 256 * i;
      int mm, kk;
      if (ALAY == kKContig) { mm = idx / TK; kk = idx % TK; } else { kk = idx / T; mm = idx % T; }
      const int m = m0 + mm, k = k0 + kk;
      float va = 0.f;
      if (m < g.M && k < g.K)
        va = ALAY == kKContig ? g.a[(int64_t)m * g.lda + k] : g.a[(int64_t)k * g.lda + m];
      As[kk][mm] = va;
      int nn, kb;
      if (BLAY == kKContig) { nn = idx / TK; kb = idx % TK; } else { kb = idx / T; nn = idx % T; }
      const int n = n0 + nn, k2 = k0 + kb;
      float vb = 0.f;
      if (n < g.N && k2 < g.K)
        vb = BLAY == kKContig ? g.b[(int64_t)n * g.ldb + k2] : g.b[(int64_t)k2 * g.ldb + n];
      Bs[kb][nn] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + ty + 16 * i, col = n0 + tx + 16 * j;
      if (row < g.M && col < g.N) epi(row, col, acc[i][j]);
    }
}

// --------------------------------------------------------------- dispatch
template <int AL, int BL, class Epi>
hipError_t run_bf16(const GemmDesc& d, const Epi& epi, hipStream_t s) {
  GemmArgs g;
  g.a = static_cast<const bf16_t*>(d.a);
  g.b = static_cast<const bf16_t*>(d.b);
  g.a2 = static_cast<const bf16_t*>(d.a2);
  g.n_split = d.n_split;
  // Spread the N tiles that run a second K pass evenly over the tile order
  // (heavy tile j at slot floor((2j+1) ntn / 2 nh), light tiles fill the rest).
  const int ntn = (d.N + BN - 1) / BN;
  const int nh = d.a2 != nullptr ? min(ntn, (d.n_split + BN - 1) / BN) : 0;
  g.use_perm = (nh > 0 && nh < ntn && ntn <= kMaxPerm) ? 1 : 0;
  if (g.use_perm) {
    int next_light = nh, j = 0;
    for (int slot = 0; slot < ntn; ++slot) {
      if (j < nh && slot == (int)(((int64_t)(2 * j + 1) * ntn) / (2 * nh))) {
        g.perm[slot] = (int16_t)j++;
      } else {
        g.perm[slot] = (int16_t)next_light++;
      }
    }
  }
  g.M = d.M; g.N = d.N; g.K = d.K; g.lda = d.lda; g.ldb = d.ldb;
  const int64_t a_elems = AL == kKContig ? (int64_t)(d.M - 1) * d.lda + d.K
                                         : (int64_t)(d.K - 1) * d.lda + d.M;
  const int64_t b_elems = BL == kKContig ? (int64_t)(d.N - 1) * d.ldb + d.K
                                         : (int64_t)(d.K - 1) * d.ldb + d.N;
  g.a_bytes = (uint32_t)(a_elems * 2);
  g.b_bytes = (uint32_t)(b_elems * 2);
  const int tiles = ((d.M + BM - 1) / BM) * ((d.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<AL, BL, Epi>), dim3(tiles), dim3(kGemmThreads), 0, s, g,
                     epi);
  return hipGetLastError();
}

template <int AL, int BL, class Epi>
hipError_t run_f32(const GemmDesc& d, const Epi& epi, hipStream_t s) {
  GemmArgsF32 g;
  g.a = static_cast<const float*>(d.a);
  g.b = static_cast<const float*>(d.b);
  g.M = d.M; g.N = d.N; g.K = d.K; g.lda = d.lda; g.ldb = d.ldb;
  const int tiles = ((d.M + 63) / 64) * ((d.N + 63) / 64);
  hipLaunchKernelGGL((gemm_f32_kernel<AL, BL, Epi>), dim3(tiles), dim3(256), 0, s, g, epi);
  return hipGetLastError();
}

template <class Epi, bool BF16>
hipError_t run_layouts(const GemmDesc& d, const Epi& epi, hipStream_t s) {
  const int key = d.a_layout * 2 + d.b_layout;
  if (BF16) {
    switch (key) {
      case 0: return run_bf16<kKContig, kKContig>(d, epi, s);
      case 1: return run_bf16<kKContig, kMNContig>(d, epi, s);
      case 2: return run_bf16<kMNContig, kKContig>(d, epi, s);
      default: return run_bf16<kMNContig, kMNContig>(d, epi, s);
    }
  } else {
    switch (key) {
      case 0: return run_f32<kKContig, kKContig>(d, epi, s);
      case 1: return run_f32<kKContig, kMNContig>(d, epi, s);
      case 2: return run_f32<kMNContig, kKContig>(d, epi, s);
      default: return run_f32<kMNContig, kMNContig>(d, epi, s);
    }
  }
}

}  // namespace

hipError_t launch_gemm_store(int dtype, const GemmDesc& d, void* c, int64_t ldc, bool c_f32,
                             hipStream_t s) {
  if (dtype == 1) {
    if (c_f32) return run_layouts<EpiStore<float>, true>(d, EpiStore<float>{(float*)c, ldc}, s);
    return run_layouts<EpiStore<bf16_t>, true>(d, EpiStore<bf16_t>{(bf16_t*)c, ldc}, s);
  }
  return run_layouts<EpiStore<float>, false>(d, EpiStore<float>{(float*)c, ldc}, s);
}

hipError_t launch_gemm_in_fwd(int dtype, const GemmDesc& d, void* qkv, void* qk_lo, void* f,
                              void* cat, int attn, int ffn, hipStream_t s) {
  if (dtype == 1) {
    EpiInFwd<bf16_t> e{(bf16_t*)qkv, (bf16_t*)qk_lo, (bf16_t*)f, (bf16_t*)cat, 3 * attn, attn,
                       ffn};
    return run_layouts<EpiInFwd<bf16_t>, true>(d, e, s);
  }
  EpiInFwd<float> e{(float*)qkv, nullptr, (float*)f, (float*)cat, 3 * attn, attn, ffn};
  return run_layouts<EpiInFwd<float>, false>(d, e, s);
}

hipError_t launch_gemm_out_fwd(int dtype, const GemmDesc& d, const void* x, int add, void* y,
                               hipStream_t s) {
  if (dtype == 1) {
    EpiOutFwd<bf16_t> e{(bf16_t*)y, (const bf16_t*)x, d.N, add};
    return run_layouts<EpiOutFwd<bf16_t>, true>(d, e, s);
  }
  EpiOutFwd<float> e{(float*)y, (const float*)x, d.N, add};
  return run_layouts<EpiOutFwd<float>, false>(d, e, s);
}

hipError_t launch_gemm_dcat(int dtype, const GemmDesc& d, const void* f, void* d_o, void* dz,
                            int attn, int ffn, hipStream_t s) {
  if (dtype == 1) {
    EpiDcat<bf16_t> e{(const bf16_t*)f, (bf16_t*)d_o, (bf16_t*)dz, attn, ffn};
    return run_layouts<EpiDcat<bf16_t>, true>(d, e, s);
  }
  EpiDcat<float> e{(const float*)f, (float*)d_o, (float*)dz, attn, ffn};
  return run_layouts<EpiDcat<float>, false>(d, e, s);
}

}  // namespace ptb
