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
// bf16 path (gfx950 MFMA): 256x256 output tile per workgroup of 8 waves (two
// per SIMD, so one wave's LDS reads, load issue and waits overlap the
// other's MFMAs), each wave a 128x64 sub-tile of 4x2
// v_mfma_f32_32x32x16_bf16 blocks with 128 fp32 accumulators; K step 64.
// Operand tiles go from memory straight into LDS (buffer loads with the LDS
// bit, no register staging) through a ring of five 32 KB slots, which keeps
// every A tile in flight for two tiles of MFMAs and every B tile for one.
// M/N-contiguous operands stay in that layout in LDS and are
// read with the transposing LDS read (ds_read_b64_tr_b16) into the K-major
// MFMA fragments.  Edges are masked by the buffer unit's range check (zero
// fill), so any M, N, K is accepted.
//
// Tile order: the hardware deals workgroups round-robin to the 8 XCDs; the
// block index is remapped so that each XCD gets a contiguous range of tiles,
// walked M-fastest within groups of 8 M-tiles, so tiles that share B columns
// run on the same XCD's L2.
//
// fp32 path: a plain LDS-tiled SIMT kernel (64x64 tile, 4x4 outputs per
// thread) with the same epilogues; it serves the fp32 workload.
#include <atomic>
#include <chrono>

#include "common.h"
#include "kernels.h"

namespace ptb {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kOpBytes = BM * BK * 2;         // one operand K tile, 32 KB (one LDS slot)
constexpr int kSlots = 5;                     // operand slots in LDS (5 x 32 KB = 160 KB)
constexpr int kSkAlign = 2;                   // stream-K ranges start on even iterations
constexpr int kWaves = 8;                     // 2 per SIMD; wave grid 2 (M) x 4 (N)
constexpr int kGemmThreads = 64 * kWaves;
constexpr int kGroupM = 8;

// --------------------------------------------------------------- epilogues
// An LDS (address space 3) view of 16 bytes, so reads of prefetched epilogue
// operands stay LDS reads (not generic loads merged with the memory path).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_uint4_t;
__device__ __forceinline__ uint4 lds_read16(const lds_uint4_t* src) {
  const u32x4_t t = *src;
  return make_uint4(t.x, t.y, t.z, t.w);
}// Each epilogue takes one accumulator value (operator(), used by the fp32
// kernel) or 8 consecutive columns of one row (used by the MFMA kernel after
// staging through LDS; col % 8 == 0, columns >= ncols dropped) in two steps:
// pre8 loads whatever else the columns need (the residual, the FC1
// pre-activation) into a Pre, and store8p combines and stores.  Splitting
// them lets a lane issue the loads of all its chunks before it waits for
// any.
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

// Eight values of an epilogue operand as loaded (bf16 stays packed until it
// is used); chunks cut by the matrix edge are read at use instead.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16_t* p, int valid) {
    if (valid >= 8) u = *reinterpret_cast<const uint4*>(p);
  }
  __device__ __forceinline__ void get(const bf16_t* p, float (&v)[8], int valid) const {
    if (valid >= 8) {
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
      get8(p, v, valid);
    }
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p, int valid) {
    if (valid >= 8) {
      a = *reinterpret_cast<const float4*>(p);
      b = *reinterpret_cast<const float4*>(p + 4);
    }
  }
  __device__ __forceinline__ void get(const float* p, float (&v)[8], int valid) const {
    if (valid >= 8) {
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      get8(p, v, valid);
    }
  }
};

template <typename T>
struct EpiStore {
  T* c;
  int64_t ldc;
  int nt = 0;  // bf16: whole chunks bypass the caches (non-temporal stores)
  __device__ __forceinline__ void operator()(int row, int col, float v) const {
    Elt<T>::st(c + (int64_t)row * ldc + col, v);
  }
  __device__ __forceinline__ void store8(int row, int col, const float (&v)[8], int ncols) const {
    T* p = c + (int64_t)row * ldc + col;
    if constexpr (sizeof(T) == 2) {
      if (nt && ncols - col >= 8) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        u32x4 u;
        u.x = pack_bf2(v[0], v[1]); u.y = pack_bf2(v[2], v[3]);
        u.z = pack_bf2(v[4], v[5]); u.w = pack_bf2(v[6], v[7]);
        __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(p));
        return;
      }
    }
    put8(p, v, ncols - col);
  }
  struct Pre {};
  static constexpr bool kOperand = false;
  __device__ __forceinline__ void pre8(int, int, Pre&, int) const {}
  __device__ __forceinline__ void store8p(int row, int col, const float (&v)[8], const Pre&,
                                          int ncols) const {
    store8(row, col, v, ncols);
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
  struct Pre {};
  static constexpr bool kOperand = false;
  __device__ __forceinline__ void pre8(int, int, Pre&, int) const {}
  __device__ __forceinline__ void store8p(int row, int col, const float (&v)[8], const Pre&,
                                          int ncols) const {
    store8(row, col, v, ncols);
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
  using Pre = Raw8<T>;
  __device__ __forceinline__ void pre8(int row, int col, Pre& p, int ncols) const {
    if (add) p.load(x + (int64_t)row * ld + col, ncols - col);
  }
  // The residual as an LDS-prefetched operand (bf16): whole 8-column chunks
  // only; a chunk cut by the matrix edge is read from memory at use.
  static constexpr bool kOperand = sizeof(T) == 2;
  __device__ __forceinline__ bool has_op(int) const { return add != 0; }
  __device__ __forceinline__ const void* op_base() const { return x; }
  __device__ __forceinline__ uint32_t op_bytes(int M) const {
    return (uint32_t)((int64_t)M * ld * sizeof(T));
  }
  __device__ __forceinline__ uint32_t op_off(int row, int col, int M, int ncols) const {
    return row < M && col + 8 <= ncols ? (uint32_t)(((int64_t)row * ld + col) * sizeof(T))
                                       : kOutOfRange;
  }
  __device__ __forceinline__ void pre8_lds(int, int col, Pre& p, int ncols,
                                           const lds_uint4_t* src) const {
    if (ncols - col >= 8) p.u = lds_read16(src);
  }
  __device__ __forceinline__ void store8p(int row, int col, const float (&v)[8], const Pre& p,
                                          int ncols) const {
    const int64_t o = (int64_t)row * ld + col;
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = v[e];
    if (add) {
      float xv[8];
      p.get(x + o, xv, ncols - col);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] += xv[e];
    }
    put8(y + o, r, ncols - col);
  }
};

// Columns < attn go to d_o [T, attn]; column attn + c (c < ffn) goes, times
// GeLU'(f[:, c]), to dz[row * dz_ld + dz_off + c].
template <typename T>
struct EpiDcat {
  const T* f;
  T* d_o;
  T* dz;
  int attn, ffn;
  int64_t dz_ld, dz_off;
  __device__ __forceinline__ void operator()(int row, int col, float v) const {
    if (col < attn) {
      Elt<T>::st(d_o + (int64_t)row * attn + col, v);
    } else {
      const int c = col - attn;
      const float fv = Elt<T>::ld(f + (int64_t)row * ffn + c);
      Elt<T>::st(dz + row * dz_ld + dz_off + c, v * gelu_grad_f(fv));
    }
  }
  // attn is a multiple of 8, so a chunk never straddles the O / FC2 border
  using Pre = Raw8<T>;
  __device__ __forceinline__ void pre8(int row, int col, Pre& p, int ncols) const {
    if (col >= attn) p.load(f + (int64_t)row * ffn + (col - attn), ncols - col);
  }
  // f stays a memory load: prefetching it into LDS one strip ahead, as the
  // residual is, measured 1-2 us slower (its reads are bandwidth-bound when
  // every CU runs this epilogue at once).
  static constexpr bool kOperand = false;
  __device__ __forceinline__ void store8p(int row, int col, const float (&v)[8], const Pre& p,
                                          int ncols) const {
    const int valid = ncols - col;
    if (col < attn) {
      put8(d_o + (int64_t)row * attn + col, v, valid);
    } else {
      const int c = col - attn;
      float fv[8], r[8];
      p.get(f + (int64_t)row * ffn + c, fv, valid);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = v[e] * gelu_grad_f(fv[e]);
      put8(dz + row * dz_ld + dz_off + c, r, valid);
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

// --------------------------------------------------------------- bf16 operand tiles
// One operand tile is 256 rows (of M or N) x 64 of K, 32 KB, and reaches LDS
// by direct buffer->LDS loads (buffer_load_dwordx4 ... lds): one wave
// instruction writes 1 KB of LDS, lane L's 16 bytes at byte 16 L, so the LDS
// layout is chosen by which global piece each lane fetches.  Out-of-range
// lanes (rows past M/N, K past the end) are steered outside the buffer and
// the load then writes zeros.
//
//   K-contiguous operand: LDS row r (128 bytes, a whole cache line of the
//   source row) holds the 64 K values of tile row r as eight 16-byte slots;
//   logical slot c sits at slot c ^ ((r>>1)&7), so the 16-byte fragment
//   reads of 16 consecutive rows hit all 64 banks.
//   M/N-contiguous operand: LDS row k (512 bytes) holds tile K row k; its 16
//   32-byte pairs (16 M/N values each) are permuted, logical pair P at
//   P ^ (2 (k&3)), so the transposing fragment reads (ds_read_b64_tr_b16,
//   4 K rows x 32 bytes per 16 lanes) hit distinct banks.
constexpr int kDmaPerOp = kOpBytes / (kGemmThreads * 16);  // DMA instructions per lane


template <int LAY>
struct DmaOperand {
  // voff[i]: byte offset of this lane's piece i in K tile 0, or kOutOfRange
  // when its row does not exist; K tile kt adds kt * kstep, which is the
  // same for every lane and goes into the scalar offset, so a full tile's
  // loads write no vector registers.  (A vector register that an
  // outstanding LDS-bound load used as its address is not rewritten before
  // that load completes, so per-tile address arithmetic would make the
  // next write to such a register wait for the load.)  kin, ikstep: K
  // index of piece 0 and the step per piece, for the masked edge tiles.
  uint32_t voff[kDmaPerOp];
  uint32_t kstep;
  int kin, ikstep;
  __device__ __forceinline__ void init(int wave, int lane, int r0, int rows, int64_t ld) {
    if (LAY == kKContig) {
      const int row = 8 * wave + (lane >> 3);   // piece 0; piece i adds 8 kWaves i rows
      kin = 8 * ((lane & 7) ^ ((row >> 1) & 7));
      ikstep = 0;
      const uint32_t base = (uint32_t)(((int64_t)(r0 + row) * ld + kin) * 2);
#pragma unroll
      for (int i = 0; i < kDmaPerOp; ++i)
        voff[i] = r0 + row + 8 * kWaves * i < rows
                      ? base + (uint32_t)(i * 8 * kWaves * ld * 2) : kOutOfRange;
      kstep = (uint32_t)(BK * 2);
    } else {
      kin = 2 * wave + (lane >> 5);             // piece 0; piece i adds 2 kWaves i K rows
      ikstep = 2 * kWaves;
      const int q = lane & 31;
      const int row = 8 * (2 * ((q >> 1) ^ (2 * (kin & 3))) + (q & 1));
      const uint32_t base = (uint32_t)(((int64_t)kin * ld + r0 + row) * 2);
#pragma unroll
      for (int i = 0; i < kDmaPerOp; ++i)
        voff[i] = r0 + row < rows ? base + (uint32_t)(i * ikstep * ld * 2) : kOutOfRange;
      kstep = (uint32_t)(BK * ld * 2);
    }
  }
  // K tile kt of the operand into LDS at `op`.  RAGGED (K is not a
  // multiple of BK): pieces at K >= klim load zeros, through per-lane
  // address selects; otherwise every tile is whole and the loads use the
  // fixed per-lane offsets plus a scalar tile offset.
  template <bool RAGGED>
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* op, int wave, int kt,
                                        int klim) const {
    if constexpr (!RAGGED) {
      const uint32_t so = (uint32_t)kt * kstep;
#pragma unroll
      for (int i = 0; i < kDmaPerOp; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(op + (i * kWaves + wave) * 1024),
                                                 16, voff[i], so, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < kDmaPerOp; ++i) {
        const bool ok = voff[i] != kOutOfRange && kt * BK + kin + i * ikstep < klim;
        const uint32_t off = ok ? voff[i] + (uint32_t)kt * kstep : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(op + (i * kWaves + wave) * 1024),
                                                 16, off, 0, 0, 0);
      }
    }
  }
};

// MFMA fragments of one K=16 step for a wave's 128 rows (4 blocks of 32):
// lane l gets rows 32 i + l%32, K values 8 (l/32) .. +8 of the step.
template <int LAY, int NF, int SLICE>
struct FragReader {
  int off[4];
  __device__ __forceinline__ void init(int lane, int wsel) {
    if (LAY == kKContig) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        off[ks] = (wsel * SLICE + (lane & 31)) * 128 +
                  16 * ((2 * ks + (lane >> 5)) ^ ((lane >> 1) & 7));
    } else {
      // ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives
      // element i%4 of the 4-value pieces addressed by lanes 4e + i/4
      // (e = 0..3), so lane j addresses K row j/4 at M/N offset 4 (j%4).
      const int g = lane >> 4, j = lane & 15;
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int pair = wsel * (SLICE / 16) + 2 * i + (g & 1);
        off[i] = (8 * (g >> 1) + (j >> 2)) * 512 + 32 * (pair ^ (2 * (j >> 2))) + 8 * (j & 3);
      }
    }
  }
  __device__ __forceinline__ void read(bf16x8_t (&f)[NF], const char* op, int ks) const {
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      // every address is the slot base plus one integer offset (a pointer
      // formed from another pointer can lose the slot's alias scope, and
      // the compiler then waits for all loads in flight before the read)
      if (LAY == kKContig) {
        f[i] = *reinterpret_cast<const bf16x8_t*>(&op[off[ks] + i * 4096]);
      } else {
        const int o = off[i] + ks * 8192;
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)&op[o]);
        const bf16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4_t*)&op[o + 2048]);
        f[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  }
};

// --------------------------------------------------------------- schedule
// Logical tile order: groups of gm M-tiles, M-fastest within a group, over
// logical N columns.  The first nh physical N-tiles also run the a2 pass
// (2 nk1 K iterations instead of nk1).  With light_first the logical columns
// list the single-pass columns first (physical nh .. ntn-1, then 0 .. nh-1),
// so that with one group (gm = ntm) every single-pass tile precedes every
// two-pass tile.  start(l) is the first iteration of logical tile l in the
// concatenation of all tiles' K iterations; locate() inverts it.
struct Sched {
  int ntm, ntn, nk1, nh, gm, light_first;
  // K iterations of physical N-tile tn
  __host__ __device__ int cost(int tn) const { return tn < nh ? 2 * nk1 : nk1; }
  __host__ __device__ int phys(int c) const {
    return !light_first ? c : (c < ntn - nh ? c + nh : c - (ntn - nh));
  }
  // iterations of one M-tile row over logical columns [0, c)
  __host__ __device__ int64_t col_prefix(int c) const {
    if (light_first) {
      const int extra = c - (ntn - nh);
      return (int64_t)nk1 * (c + (extra > 0 ? extra : 0));
    }
    return (int64_t)nk1 * (c + (c < nh ? c : nh));
  }
  __host__ __device__ int group_size(int first_m) const {
    return ntm - first_m < gm ? ntm - first_m : gm;
  }
  __host__ __device__ void logical(int l, int& tm, int& c) const {
    const int group = l / (gm * ntn), first_m = group * gm;
    const int gsize = group_size(first_m), in = l - group * gm * ntn;
    c = in / gsize;
    tm = first_m + in % gsize;
  }
  __host__ __device__ void tile(int l, int& tm, int& tn) const {
    int c;
    logical(l, tm, c);
    tn = phys(c);
  }
  __host__ __device__ int64_t start(int l) const {
    if (l >= ntm * ntn) return (int64_t)ntm * col_prefix(ntn);
    int tm, c;
    logical(l, tm, c);
    const int first_m = tm - tm % gm;
    return (int64_t)first_m * col_prefix(ntn) + (int64_t)group_size(first_m) * col_prefix(c) +
           (int64_t)(tm - first_m) * cost(phys(c));
  }
  __host__ __device__ void locate(int64_t it, int& l, int& koff) const {
    const int64_t row = col_prefix(ntn);
    const int ngroups = (ntm + gm - 1) / gm;
    int group = (int)(it / (gm * row));
    if (group >= ngroups) group = ngroups - 1;
    const int first_m = group * gm, gsize = group_size(first_m);
    int64_t rem = it - (int64_t)first_m * row;
    // the logical columns form two runs of equal cost: n0 columns of c0
    // iterations, then the rest of c1
    const int n0 = light_first ? ntn - nh : nh;
    const int c0 = light_first ? nk1 : 2 * nk1, c1 = light_first ? 2 * nk1 : nk1;
    const int64_t first_run = (int64_t)gsize * c0 * n0;
    int c, cost_c;
    if (rem < first_run) {
      cost_c = c0;
      c = (int)(rem / ((int64_t)gsize * c0));
      rem -= (int64_t)c * gsize * c0;
    } else {
      cost_c = c1;
      rem -= first_run;
      const int q = (int)(rem / ((int64_t)gsize * c1));
      c = n0 + q;
      rem -= (int64_t)q * gsize * c1;
    }
    const int r = (int)(rem / cost_c);
    koff = (int)(rem - (int64_t)r * cost_c);
    l = group * gm * ntn + c * gsize + r;
  }
};

// a2 (optional, same layout and leading dimension as a): output tiles whose
// first column lies below n_split accumulate a second K pass over a2 with
// the same B, i.e. C = (A + A2) B^T there.  The input projection uses it to
// form q and k from the LayerNorm output split into its bf16 value and bf16
// residual, so the attention scores do not inherit the rounding of xn.
//
// Two schedules.  sk == 0: workgroup b computes tile tile_coords(b) whole.
// sk == 1 (persistent, `grid` workgroups, one per CU): the first dp_tiles
// logical tiles are dealt out whole; the K iterations of the remaining tiles
// are split into `grid` equal contiguous ranges (stream-K), so every CU gets
// the same amount of work when the tile count is not a multiple of the CU
// count.  A range that covers only part of a tile writes its fp32 partial
// tile to ws and counts itself in the tile's arrival counter; the workgroup
// that completes the count sums the tile's partials from ws in K order and
// runs the epilogue, so results do not depend on timing or on which
// contributor finishes last.  With several whole rounds of tiles and no
// split (dp_tiles = every tile, an empty range), sk == 1 simply walks each
// CU's tiles in one persistent launch.
struct GemmArgs {
  const bf16_t* a;
  const bf16_t* b;
  const bf16_t* a2;
  int M, N, K;
  int n_split;
  int64_t lda, ldb;
  uint32_t a_bytes, b_bytes;
  Sched sc;
  int sk, grid, dp_tiles;
  int64_t sk_base, sk_iters;
  float* ws;
  unsigned long long* arrive;  // one counter per split tile (logical tile - dp_tiles)
  unsigned long long tag;      // 48-bit launch tag
  int use_perm;
  int16_t perm[kMaxPerm];  // N-tile order (when use_perm, sk == 0)
};
constexpr int kPartialFloats = BM * BN;  // one partial tile in ws
// Cache policy of the partial-tile accesses: device scope (sc1), coherent
// across the XCDs' L2s.
constexpr int kCpolDevice = 16;

// First iteration of stream-K worker w (w == grid: end of the range);
// rounded down to a multiple of kSkAlign.
__host__ __device__ inline int64_t sk_lo(const GemmArgs& g, int w) {
  if (w >= g.grid) return g.sk_base + g.sk_iters;
  return g.sk_base + (((int64_t)w * g.sk_iters / g.grid) & ~(int64_t)(kSkAlign - 1));
}
// The stream-K worker whose range holds iteration it.
__device__ inline int sk_owner(const GemmArgs& g, int64_t it) {
  int w = (int)((it - g.sk_base) * g.grid / g.sk_iters);
  w = w < 0 ? 0 : (w > g.grid - 1 ? g.grid - 1 : w);
  while (w > 0 && sk_lo(g, w) > it) --w;
  while (w < g.grid - 1 && sk_lo(g, w + 1) <= it) ++w;
  return w;
}
// ws slot of worker w's segment of a tile starting at iteration s: its first
// segment (which may start inside the tile) or its last one.
__device__ inline int sk_slot(const GemmArgs& g, int w, int64_t s) {
  return sk_lo(g, w) >= s ? 2 * w : 2 * w + 1;
}

// Counts one contribution to a split tile and returns true for the one that
// completes it (n contributions in all).  Counter word: launch tag in bits
// 63..16, contributions so far in bits 15..0; a word carrying another tag
// (an earlier launch, or memory never used as a counter) counts as none.
// The completing contribution stores 0, so the counters also stay valid
// when a captured launch is replayed with the same tag.  Every failed
// exchange means another contributor's exchange succeeded, so the loop ends
// after at most n rounds; the bound only guards against foreign writes.
// The exchange itself is device-scope and relaxed: the partials it guards
// are written and read with device-scope (sc1) accesses, the writer waits
// for its stores to complete before counting, and the reader loads only
// after the verdict, so no cache-wide release or acquire is needed.
__device__ __forceinline__ bool arrive_last(unsigned long long* c, unsigned long long tag, int n) {
  unsigned long long old = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int tries = 0; tries < 4096; ++tries) {
    const unsigned long long have = (old >> 16) == tag ? (old & 0xffffull) : 0ull;
    const bool last = (int)have + 1 >= n;
    const unsigned long long next = last ? 0ull : (tag << 16) | (have + 1);
    if (__hip_atomic_compare_exchange_strong(c, &old, next, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return last;
  }
  return false;
}

// 8 MFMAs of one K=16 step: the wave's 128x64 accumulators.
__device__ __forceinline__ void mma_step(f32x16_t (&acc)[4][2], const bf16x8_t (&fa)[4],
                                         const bf16x8_t (&fb)[2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
}

// Scheduling of one phase (masks: 0x008 MFMA, 0x020 memory read, 0x100 LDS
// read): the 16 MFMAs, each followed by an LDS read on every RS-th one (NR in
// all) and a memory read on every VS-th one (NV in all), closed by a full
// scheduling barrier.
template <int NR, int NV, int VS>
__device__ __forceinline__ void interleave() {
  static_assert(NR <= 16 && NV * VS <= 8, "fits in one phase");
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (i + 8 < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (i % VS == VS - 1 && i / VS < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Wait until at most VM memory instructions of this wave are outstanding and
// its LDS reads are done, then barrier.  (A plain __syncthreads would wait
// for every outstanding load, draining the pipeline.)
template <int VM>
__device__ __forceinline__ void wait_barrier() {
  static_assert(VM < 64, "vmcnt field");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Epilogue of one row of two 32x32 accumulator blocks (a = acc[i][0..1]):
// each wave stages its 32x64 strip in its own LDS area (fp32; block j at
// word j*kStageBlk + 4j so the row-chunk reads of the two blocks fall on
// different banks) with a short fully unrolled loop, then re-reads it as
// 8-column row chunks (8 rows x 64 columns per wave instruction, four per
// lane).  A lane first gathers its four chunks and issues the epilogue's own
// loads for all of them (pre8), then combines and stores (store8p), so those
// loads are in flight together instead of one after another.  Every lane
// issues 16-byte stores.  Contains two workgroup barriers.
constexpr int kStageRow = 36, kStageBlk = 1216;
template <class Epi>
__device__ __forceinline__ void epilogue_strip(const f32x16_t (&a)[2], float* stage, int row0,
                                               int col0, int lane, int M, int N, const Epi& epi,
                                               bool use_op = false, const char* opbuf = nullptr,
                                               bool op_last = false) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float* blk = stage + j * kStageBlk + j * 4;
#pragma unroll
    for (int r = 0; r < 16; ++r) blk[mfma32_row(r, lane) * kStageRow + (lane & 31)] = a[j][r];
  }
  if constexpr (Epi::kOperand) {
    // prefetched operand: this strip's chunks (the wave's own LDS-bound
    // loads) have landed once at most the next strip's four loads remain
    if (use_op) {
      if (op_last)
        __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0) lgkmcnt(0)
      else
        __builtin_amdgcn_s_waitcnt(4 | (7 << 4));  // vmcnt(4) lgkmcnt(0)
    }
  }
  __syncthreads();
  constexpr int kChunks = 32 * 8 / 64;  // 8-column chunks of the 32x64 strip per lane
  float v[kChunks][8];
  typename Epi::Pre pre[kChunks];
#pragma unroll
  for (int q = 0; q < kChunks; ++q) {
    const int c = lane + 64 * q;
    const int rr = c >> 3, jc = c & 7, j = jc >> 2, c8 = (jc & 3) * 8;
    const float* src = stage + j * kStageBlk + j * 4 + rr * kStageRow + c8;
    const float4 lo = *reinterpret_cast<const float4*>(src);
    const float4 hi = *reinterpret_cast<const float4*>(src + 4);
    v[q][0] = lo.x; v[q][1] = lo.y; v[q][2] = lo.z; v[q][3] = lo.w;
    v[q][4] = hi.x; v[q][5] = hi.y; v[q][6] = hi.z; v[q][7] = hi.w;
    const int row = row0 + rr, col = col0 + j * 32 + c8;
    if (row < M && col < N) {
      if constexpr (Epi::kOperand) {
        if (use_op)
          epi.pre8_lds(row, col, pre[q], N, (const lds_uint4_t*)(opbuf + q * 1024 + lane * 16));
        else
          epi.pre8(row, col, pre[q], N);
      } else {
        epi.pre8(row, col, pre[q], N);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < kChunks; ++q) {
    const int c = lane + 64 * q;
    const int rr = c >> 3, jc = c & 7, j = jc >> 2, c8 = (jc & 3) * 8;
    const int row = row0 + rr, col = col0 + j * 32 + c8;
    if (row < M && col < N) epi.store8p(row, col, v[q], pre[q], N);
  }
  __syncthreads();
}

// LDS-bound loads of one strip's epilogue operand chunks (the 32 x 64 strip
// at row0, col0, in the chunk order epilogue_strip reads) into this wave's
// 4 KB area `dst`: four wave instructions, lane L's chunk q at
// dst + 1024 q + 16 L.  Chunks without an operand load zeros.
template <class Epi>
struct OperandLoads {
  __amdgpu_buffer_rsrc_t rs;
  __device__ __forceinline__ void init(const Epi& epi, int M) {
    rs = make_rsrc(epi.op_base(), epi.op_bytes(M));
  }
  __device__ __forceinline__ void issue(const Epi& epi, char* dst, int row0, int col0, int lane,
                                        int M, int N) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = lane + 64 * q;
      const int rr = c >> 3, jc = c & 7, j = jc >> 2, c8 = (jc & 3) * 8;
      // (the offset goes through a local: passing the call itself as the
      // builtin's argument made the compiler drop the host launch stubs)
      const uint32_t vo = epi.op_off(row0 + rr, col0 + j * 32 + c8, M, N);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + q * 1024), 16, vo, 0, 0, 0);
    }
  }
};

// Offset (floats) of this lane's accumulators acc[i][j][4 r4 .. 4 r4 + 3] in
// a partial tile: one 1 KB run per (wave, i, j, r4), so each store or load
// instruction of a wave is contiguous.
__device__ __forceinline__ int partial_off(int wave, int i, int j, int r4, int lane) {
  return ((((wave * 4 + i) * 2 + j) * 4 + r4) * 64 + lane) * 4;
}

// Main loop of one segment (K iterations kb .. ke of a tile; iterations
// nk1.. of a two-pass tile read a2).  Operand K tiles A_t and B_t (32 KB
// each) rotate through five LDS slots in the order A0 B0 A1 B1 A2 B2 ...,
// so while tile t is multiplied, tile t+1 is resident or landing and A_{t+2}
// is in flight: A tiles are loaded two tiles ahead of use and B tiles one,
// which halves the data each per-tile barrier waits for.  Each tile is four
// phases of 16 MFMAs (one K=16 step each); every phase reads the next step's
// fragments while it multiplies.  The first phase issues A_{t+2} into B_{t-1}'s
// slot; after the third, each wave waits for its own loads of tile t+1 (all
// but A_{t+2}) and the workgroup meets at the tile's only barrier; the
// fourth phase reads tile t+1's first fragments and issues B_{t+2} into
// A_t's slot.  The slot pattern repeats every five tiles, so the loop is
// unrolled by five and every LDS address is static.  Whole groups of five
// run while every load they issue is a real tile (t + 2 < ke); the last
// one to six tiles then go through a copy of the tile step that loads only
// tiles before ke and waits for exactly the loads in flight (all of them
// when none is issued ahead).  RAGGED: K is not a multiple of BK, so the
// last K tile masks its loads lane by lane.
template <int ALAY, int BLAY, bool RAGGED, class Epi>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_bf16_kernel(GemmArgs g, Epi epi) {
  // one array per slot, so the compiler sees that loads into one slot do
  // not alias fragment reads from another
  __shared__ __attribute__((aligned(1024))) char s0[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char s1[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char s2[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char s3[kOpBytes];
  __shared__ __attribute__((aligned(1024))) char s4[kOpBytes];
  static_assert(kSlots == 5, "slot arrays");
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, g.a_bytes);
  const __amdgpu_buffer_rsrc_t ra2 = make_rsrc(g.a2 != nullptr ? g.a2 : g.a, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.b, g.b_bytes);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wm = wave >> 2, wn = wave & 3;
  FragReader<ALAY, 4, 128> fra;
  FragReader<BLAY, 2, 64> frb;
  fra.init(lane, wm);
  frb.init(lane, wn);
  float* stage = reinterpret_cast<float*>((wave < 3 ? s0 : wave < 6 ? s1 : s2) +
                                          (wave % 3) * (2 * kStageBlk * 4));
  static_assert(3 * 2 * kStageBlk * 4 <= kOpBytes, "epilogue staging");
  constexpr int kReads = (ALAY == kKContig ? 4 : 8) + (BLAY == kKContig ? 2 : 4);
  const int nk1 = g.sc.nk1;

  // segment source: whole tiles first, then (sk) this worker's range
  const int b = blockIdx.x, per = g.grid >> 3;
  const int gl = (b & 7) * per + (b >> 3);  // sk: XCD-contiguous worker index
  // sk: XCD x owns logical tiles [x dpx, (x + 1) dpx) of the whole-tile
  // part; its workers take them round-robin
  const int dpx = g.dp_tiles >> 3, local = b >> 3;
  int dp_left = !g.sk ? 1 : (local < dpx ? (dpx - local + per - 1) / per : 0);
  int dp_next = (b & 7) * dpx + local;
  int64_t it = g.sk ? sk_lo(g, gl) : 0;
  const int64_t it_end = g.sk ? sk_lo(g, gl + 1) : 0;
  bool first_sk = true;
  for (;;) {
    int tm, tn, kb, ke, slot = -1, lt = 0;
    if (dp_left > 0) {
      if (g.sk) {
        g.sc.tile(dp_next, tm, tn);
        dp_next += per;
      } else {
        tile_coords(b, g.sc.ntm, g.sc.ntn, g.use_perm ? g.perm : nullptr, tm, tn);
      }
      --dp_left;
      kb = 0;
      ke = g.sc.cost(tn);
    } else if (it < it_end) {
      int koff;
      g.sc.locate(it, lt, koff);
      g.sc.tile(lt, tm, tn);
      const int c = g.sc.cost(tn);
      const int seg = (int)(it_end - it < (int64_t)(c - koff) ? it_end - it : (int64_t)(c - koff));
      kb = koff;
      ke = koff + seg;
      if (kb > 0 || ke < c) slot = first_sk ? 2 * gl : 2 * gl + 1;
      first_sk = false;
      it += seg;
    } else {
      break;
    }
    const int m0 = tm * BM, n0 = tn * BN;
    DmaOperand<ALAY> da;
    DmaOperand<BLAY> db;
    da.init(wave, lane, m0, g.M, g.lda);
    db.init(wave, lane, n0, g.N, g.ldb);
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // (only the prologue may load past ke: tile kb + 1 of a one-tile
    // segment, which reloads tile ke - 1 and is drained by its wait)
    auto issue_a = [&](char* st, int t) {
      const int u = t < ke ? t : ke - 1;
      const bool second = u >= nk1;
      da.template issue<RAGGED>(second ? ra2 : ra, st, wave, second ? u - nk1 : u, g.K);
    };
    auto issue_b = [&](char* st, int t) {
      const int u = t < ke ? t : ke - 1;
      db.template issue<RAGGED>(rb, st, wave, u >= nk1 ? u - nk1 : u, g.K);
    };
    bf16x8_t fa[2][4], fb[2][2];
    // Tile t: A_t in slot ca, B_t in cb, tile t+1 in na / nb; sa is
    // B_{t-1}'s slot, which takes A_{t+2}.  (The loads sit inside the
    // branches so they interleave with the MFMAs.)
    auto tile = [&](char* ca, char* cb, char* na, char* nb, char* sa, int t) {
      const bool live = t < ke;
      if (live) {
        issue_a(sa, t + 2);
        fra.read(fa[1], ca, 1);
        frb.read(fb[1], cb, 1);
        mma_step(acc, fa[0], fb[0]);
        interleave<kReads, kDmaPerOp, 2>();
        fra.read(fa[0], ca, 2);
        frb.read(fb[0], cb, 2);
        mma_step(acc, fa[1], fb[1]);
        interleave<kReads, 0, 1>();
        fra.read(fa[1], ca, 3);
        frb.read(fb[1], cb, 3);
        mma_step(acc, fa[0], fb[0]);
        interleave<kReads, 0, 1>();
      }
      // A_{t+1} and B_{t+1} have landed (A_{t+2}, issued last, may still be
      // in flight) and every wave is done reading tile t
      wait_barrier<kDmaPerOp>();
      fra.read(fa[0], na, 0);
      frb.read(fb[0], nb, 0);
      if (live) {
        issue_b(ca, t + 2);
        mma_step(acc, fa[1], fb[1]);
        interleave<kReads, kDmaPerOp, 1>();
      }
    };

    issue_a(s0, kb);
    issue_b(s1, kb);
    issue_a(s2, kb + 1);
    issue_b(s3, kb + 1);
    wait_barrier<2 * kDmaPerOp>();
    fra.read(fa[0], s0, 0);
    frb.read(fb[0], s1, 0);
    // The last tiles of the segment (at most six, starting at the first slot
    // of the pattern): only tiles before ke are loaded, and each wait counts
    // exactly the loads in flight.
    auto tile_end = [&](char* ca, char* cb, char* na, char* nb, char* sa, int t) {
      if (t >= ke) return;  // uniform over the workgroup
      const bool ahead = t + 2 < ke;
      if (ahead) issue_a(sa, t + 2);
      fra.read(fa[1], ca, 1);
      frb.read(fb[1], cb, 1);
      mma_step(acc, fa[0], fb[0]);
      interleave<kReads, kDmaPerOp, 2>();
      fra.read(fa[0], ca, 2);
      frb.read(fb[0], cb, 2);
      mma_step(acc, fa[1], fb[1]);
      interleave<kReads, 0, 1>();
      fra.read(fa[1], ca, 3);
      frb.read(fb[1], cb, 3);
      mma_step(acc, fa[0], fb[0]);
      interleave<kReads, 0, 1>();
      if (ahead)
        wait_barrier<kDmaPerOp>();
      else
        wait_barrier<0>();
      if (t + 1 < ke) {
        fra.read(fa[0], na, 0);
        frb.read(fb[0], nb, 0);
      }
      if (ahead) issue_b(ca, t + 2);
      mma_step(acc, fa[1], fb[1]);
      interleave<kReads, kDmaPerOp, 1>();
    };
    int t = kb;
    for (; t + kSlots + 1 < ke; t += kSlots) {  // every load of the group is a real tile
      tile(s0, s1, s2, s3, s4, t);
      tile(s2, s3, s4, s0, s1, t + 1);
      tile(s4, s0, s1, s2, s3, t + 2);
      tile(s1, s2, s3, s4, s0, t + 3);
      tile(s3, s4, s0, s1, s2, t + 4);
    }
    tile_end(s0, s1, s2, s3, s4, t);
    tile_end(s2, s3, s4, s0, s1, t + 1);
    tile_end(s4, s0, s1, s2, s3, t + 2);
    tile_end(s1, s2, s3, s4, s0, t + 3);
    tile_end(s3, s4, s0, s1, s2, t + 4);
    tile_end(s0, s1, s2, s3, s4, t + 5);
    __builtin_amdgcn_s_waitcnt(0);  // no load may still be writing LDS
    __syncthreads();

    if (slot < 0) {
      // An epilogue operand (the residual, bf16) comes into the idle slots
      // s3 / s4 with LDS-bound loads one strip ahead: each lane loads exactly
      // the four 16-byte chunks it combines later, so it reads back its own
      // data (4 KB per wave and strip, four loads per lane), and a strip
      // waits with vmcnt(4) for its own chunks.
      bool pf = false;
      if constexpr (Epi::kOperand) pf = epi.has_op(n0);
      char* const ob0 = s3 + wave * 4096;
      char* const ob1 = s4 + wave * 4096;
      const int orow = m0 + wm * 128, ocol = n0 + wn * 64;
      if constexpr (Epi::kOperand) {
        if (pf) {
          OperandLoads<Epi> ol;
          ol.init(epi, g.M);
          ol.issue(epi, ob0, orow, ocol, lane, g.M, g.N);
          ol.issue(epi, ob1, orow + 32, ocol, lane, g.M, g.N);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (Epi::kOperand) {
          if (pf && i >= 1 && i <= 2) {
            OperandLoads<Epi> ol;
            ol.init(epi, g.M);
            ol.issue(epi, (i & 1) ? ob0 : ob1, orow + (i + 1) * 32, ocol, lane, g.M, g.N);
          }
        }
        epilogue_strip(acc[i], stage, m0 + wm * 128 + i * 32, n0 + wn * 64, lane, g.M, g.N, epi,
                       pf, (i & 1) ? ob1 : ob0, i == 3);
      }
    } else {
      // Partials move with device-scope (sc1) buffer stores and loads, which
      // other XCDs see without a writeback or invalidation of the whole L2.
      const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.ws, (uint32_t)kGemmPartialBytes);
      const uint32_t so =
          __builtin_amdgcn_readfirstlane((uint32_t)slot * (uint32_t)(kPartialFloats * 4));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4_t v = {acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2],
                               acc[i][j][4 * r4 + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(v, rw, (uint32_t)partial_off(wave, i, j, r4, lane) * 4,
                                                   so, kCpolDevice);
          }
      // Count the partial once every wave's stores have completed.  Every
      // LDS slot is idle here (the loads were drained above and the next
      // segment's first loads come after a barrier), so slot s4 carries the
      // verdict to the workgroup.
      const int64_t ts = g.sc.start(lt), te = g.sc.start(lt + 1);
      const int w0 = sk_owner(g, ts), w1 = sk_owner(g, te - 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      int* verdict = reinterpret_cast<int*>(s4);
      if (threadIdx.x == 0) {
        int n = 0;
        for (int w = w0; w <= w1; ++w) n += sk_lo(g, w) != sk_lo(g, w + 1);
        *verdict = arrive_last(g.arrive + (lt - g.dp_tiles), g.tag, n) ? 1 : 0;
      }
      __syncthreads();
      if (*verdict != 0) {
        // The tile is complete: add its partials in worker (= K) order (this
        // workgroup's own read back like the others, so the accumulators are
        // free) and run the epilogue.
#pragma unroll 1
        for (int i = 0; i < 4; ++i) {
          f32x16_t a[2];
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) a[j][r] = 0.f;
#pragma unroll 1
          for (int w = w0; w <= w1; ++w) {
            if (sk_lo(g, w) == sk_lo(g, w + 1)) continue;
            const uint32_t src = __builtin_amdgcn_readfirstlane(
                (uint32_t)sk_slot(g, w, ts) * (uint32_t)(kPartialFloats * 4));
            f32x4_t v[8];
#pragma unroll
            for (int c = 0; c < 8; ++c)
              v[c] = __builtin_amdgcn_raw_buffer_load_b128(
                  rw, (uint32_t)partial_off(wave, i, c >> 2, c & 3, lane) * 4, src, kCpolDevice);
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
              for (int e = 0; e < 4; ++e) a[c >> 2][4 * (c & 3) + e] += v[c][e];
          }
          epilogue_strip(a, stage, m0 + wm * 128 + i * 32, n0 + wn * 64, lane, g.M, g.N, epi);
        }
      }
    }
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
// Workgroups of a persistent launch: the CU count of the current device,
// rounded down to a multiple of the 8 XCDs, at most kSkMaxGrid (0 if unknown).
// The per-device cache is atomic: racing first calls store the same value.
int persistent_grid() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = cached[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cus = (cus < kSkMaxGrid ? cus : kSkMaxGrid) & ~7;
    c = cus > 0 ? cus : -1;
    cached[dev].store(c, std::memory_order_relaxed);
  }
  return c > 0 ? c : 0;
}

// A 48-bit tag per split launch, so arrival counters left by earlier
// launches (or never initialised) read as empty.  Starts at a clock-derived
// value so that a fresh process does not reuse the tags of an earlier one.
unsigned long long next_launch_tag() {
  static std::atomic<unsigned long long> counter{
      (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761ull};
  return counter.fetch_add(1, std::memory_order_relaxed) & 0xffffffffffffull;
}

template <int AL, int BL, class Epi>
hipError_t run_bf16(const GemmDesc& d, const Epi& epi, hipStream_t s) {
  GemmArgs g;
  g.a = static_cast<const bf16_t*>(d.a);
  g.b = static_cast<const bf16_t*>(d.b);
  g.a2 = static_cast<const bf16_t*>(d.a2);
  g.n_split = d.n_split;
  g.M = d.M; g.N = d.N; g.K = d.K; g.lda = d.lda; g.ldb = d.ldb;
  const int64_t a_elems = AL == kKContig ? (int64_t)(d.M - 1) * d.lda + d.K
                                         : (int64_t)(d.K - 1) * d.lda + d.M;
  const int64_t b_elems = BL == kKContig ? (int64_t)(d.N - 1) * d.ldb + d.K
                                         : (int64_t)(d.K - 1) * d.ldb + d.N;
  g.a_bytes = (uint32_t)(a_elems * 2);
  g.b_bytes = (uint32_t)(b_elems * 2);
  const int ntm = (d.M + BM - 1) / BM, ntn = (d.N + BN - 1) / BN;
  const int nh = d.a2 != nullptr ? min(ntn, (d.n_split + BN - 1) / BN) : 0;
  g.sc = Sched{ntm, ntn, (d.K + BK - 1) / BK, nh, kGroupM, 0};
  const int tiles = ntm * ntn;
  g.ws = static_cast<float*>(d.ws);
  g.use_perm = 0;
  g.sk = 0;
  g.grid = 8;
  g.dp_tiles = 0;
  g.sk_base = g.sk_iters = 0;
  g.arrive = nullptr;
  g.tag = 0;

  // Stream-K when whole tiles per CU would leave more than a tenth of the
  // machine idle: compare the ideal share of K iterations per CU with the
  // busiest CU of the one-tile-per-workgroup schedule (a two-pass tile
  // counts twice, and alone takes two units).
  const int G = persistent_grid();
  const int64_t total = g.sc.start(tiles);
  if (G >= 8 && g.ws != nullptr && d.ws_bytes >= kGemmWsBytes && total >= 2 * (int64_t)G * kSkAlign) {
    const int64_t units = tiles + (int64_t)nh * ntm;  // in single-pass-tile units
    int64_t dp_rounds = (units + G - 1) / G;
    if (nh > 0 && dp_rounds < 2) dp_rounds = 2;
    const int64_t dp_time = dp_rounds * g.sc.nk1;
    if ((double)total / G < 0.9 * (double)dp_time) {
      g.sk = 1;
      g.grid = G;
      g.dp_tiles = (tiles / G) * G;  // whole waves of tiles, the remainder split
      if (nh > 0) {
        // Single-pass tiles first, whole (their loads stay aligned across the
        // CUs of an XCD, so they share operand panels in L2), the two-pass
        // tiles split over all CUs; taken when its busiest CU is within a
        // tenth of the even split of everything.
        Sched lf = g.sc;
        lf.light_first = 1;
        lf.gm = ntm;
        const int dp = (ntm * (ntn - nh)) & ~7;
        const int64_t per = G / 8, dpx = dp / 8;
        const int64_t busiest = (dpx + per - 1) / per * lf.nk1 + (total - lf.start(dp)) / G;
        if ((double)busiest <= 1.1 * (double)total / G) {
          g.sc = lf;
          g.dp_tiles = dp;
        } else {
          g.dp_tiles = 0;
        }
      }
      g.sk_base = g.sc.start(g.dp_tiles);
      g.sk_iters = total - g.sk_base;
      if (tiles - g.dp_tiles > kSkMaxSplitTiles) {
        g.sk = 0;  // more split tiles than arrival counters
        g.sc = Sched{ntm, ntn, (d.K + BK - 1) / BK, nh, kGroupM, 0};
        g.grid = 8;
        g.dp_tiles = 0;
        g.sk_base = g.sk_iters = 0;
      } else {
        g.arrive = reinterpret_cast<unsigned long long*>(static_cast<char*>(d.ws) + kGemmPartialBytes);
        g.tag = next_launch_tag();
      }
    }
  }
  // Several rounds of whole tiles: run them persistently (one workgroup per
  // CU walking its tiles in the same order), which saves a workgroup launch
  // per tile; the split range is left empty.
  if (!g.sk && nh == 0 && G >= 8 && tiles > G && tiles % 8 == 0) {
    g.sk = 1;
    g.grid = G;
    g.dp_tiles = tiles;
    g.sk_base = total;
    g.sk_iters = 0;
  }
  if (!g.sk) {
    // Spread the N tiles that run a second K pass evenly over the tile order
    // (heavy tile j at slot floor((2j+1) ntn / 2 nh), light tiles fill the rest).
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
    if (d.K % BK == 0)
      hipLaunchKernelGGL((gemm_bf16_kernel<AL, BL, false, Epi>), dim3(tiles), dim3(kGemmThreads),
                         0, s, g, epi);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<AL, BL, true, Epi>), dim3(tiles), dim3(kGemmThreads),
                         0, s, g, epi);
    return hipGetLastError();
  }
  if (d.K % BK == 0)
    hipLaunchKernelGGL((gemm_bf16_kernel<AL, BL, false, Epi>), dim3(g.grid), dim3(kGemmThreads),
                       0, s, g, epi);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<AL, BL, true, Epi>), dim3(g.grid), dim3(kGemmThreads), 0,
                       s, g, epi);
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
                             hipStream_t s, bool streaming) {
  if (dtype == 1) {
    if (c_f32) return run_layouts<EpiStore<float>, true>(d, EpiStore<float>{(float*)c, ldc}, s);
    return run_layouts<EpiStore<bf16_t>, true>(
        d, EpiStore<bf16_t>{(bf16_t*)c, ldc, streaming ? 1 : 0}, s);
  }
  return run_layouts<EpiStore<float>, false>(d, EpiStore<float>{(float*)c, ldc}, s);
}

hipError_t launch_gemm_in_fwd(int dtype, const GemmDesc& d, void* qkv, void* qk_lo, void* f,
                              void* cat, int attn, int ffn, int qkv_cols, hipStream_t s) {
  if (dtype == 1) {
    EpiInFwd<bf16_t> e{(bf16_t*)qkv, (bf16_t*)qk_lo, (bf16_t*)f, (bf16_t*)cat, qkv_cols, attn,
                       ffn};
    return run_layouts<EpiInFwd<bf16_t>, true>(d, e, s);
  }
  EpiInFwd<float> e{(float*)qkv, nullptr, (float*)f, (float*)cat, qkv_cols, attn, ffn};
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
                            int attn, int ffn, int64_t dz_ld, int64_t dz_off, hipStream_t s) {
  if (dtype == 1) {
    EpiDcat<bf16_t> e{(const bf16_t*)f, (bf16_t*)d_o, (bf16_t*)dz, attn, ffn, dz_ld, dz_off};
    return run_layouts<EpiDcat<bf16_t>, true>(d, e, s);
  }
  EpiDcat<float> e{(const float*)f, (float*)d_o, (float*)dz, attn, ffn, dz_ld, dz_off};
  return run_layouts<EpiDcat<float>, false>(d, e, s);
}

}  // namespace ptb
