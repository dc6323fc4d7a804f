// device_common.hpp -- shared device helpers for the gfx950 attention-backward
// kernels: element types, 32x32 MFMA wrappers, fragment layouts, LDS tiles,
// the chunk prefetcher, mask evaluation and the workgroup -> tile mapping.
//
// Fragment conventions (wave64, 32x32 MFMA).  lane = 0..63, l32 = lane & 31,
// half = lane >> 5.  One MFMA step contracts KS k-values; every lane holds
// KL = KS / 2 consecutive ones:
//   A[M=32][K]: lane holds A[l32][s*KS + half*KL + e], e < KL
//   B[K][N=32]: lane holds B[s*KS + half*KL + e][l32]
//   C[32][32] : acc[r] = C[kr(r, half)][l32], kr(r, h) = 8*(r/4) + 4*h + r%4
// bf16 uses v_mfma_f32_32x32x16_bf16 (KS = 16, KL = 8); fp32 uses
// v_mfma_f32_32x32x2_f32 (KS = 2, KL = 1).
//
// "C reuse": a C tile whose lanes hold column n = l32 and rows kr(r, half) is
// fed straight back as the B operand of a product that contracts over those
// rows, with the rows permuted consistently on both operands: in bf16 step s,
// element e of lane (n, half) stands for row kidx(s, half, e) =
// 16 s + 8 (e / 4) + 4 half + e % 4 (which is kr(8 s + e, half)); in fp32 step
// r the lane stands for row kr(r, half).  The matching A operand reads those
// rows of one column from LDS: with ds_read_b64_tr_b16 (bf16) or a plain
// element read (fp32).  No register shuffles are needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBig = 1 << 30;  // "no limit" for the index mask offsets

// Mask evaluation modes the kernels are instantiated for.
enum { MODE_INDEX = 0, MODE_KEYPAD = 1, MODE_BIAS = 2 };

struct DenseParams {
  const void *q, *k, *v, *dy;
  void *dq, *dk, *dv;
  int64_t qs[3], ks[3], vs[3], dys[3], dqs[3], dks[3], dvs[3];  // (b, s, h) strides
  const float *mask;
  int64_t ms[4];  // (b, h, i, j) strides
  float thr;
  float scale;       // natural scale, multiplies dS
  float scale_log2;  // scale * log2(e), turns Q.K into a log2-domain score
  float inv_scale_log2;  // 1 / scale_log2
  int B, H, Sq, Sk;
  int Hkv, G;  // K / V heads and the query heads per K / V head (H = Hkv * G)
  // Index rule: key j is visible to query i iff lo_off <= j - i <= hi_off
  // (and i < Sq, j < Sk).  Causal: hi_off = max(Sk - Sq, 0); window:
  // lo_off = hi_off - w; otherwise +-kBig.
  int lo_off, hi_off;
  int need_dk, need_dv;
  int nblk;  // tiles along the blocked sequence axis
  // [B * H * Sq] each.  st_nls = -lse2 / scale_log2 = -(m + ln l) / scale
  // (-inf / scale for a row that sees nothing), so that st_nls * scale_log2 is
  // the log2-domain offset of the row's probabilities.
  float *st_m, *st_l, *st_delta, *st_nls;
  // A forward's saved statistics (dQ kernel only; fo == nullptr otherwise):
  // its natural log-sum-exp [B * H * Sq] and output O (strided like dY).  The
  // dQ kernel then forms delta and -lse2 itself and writes them to st_delta /
  // st_nls for the dK / dV kernel that follows.
  const void *fo;
  const float *flse;
  int64_t fos[3];
  // Split form of the row-statistics and dQ passes (ws_split != nullptr): the
  // key axis in pieces of piece_chunks 32-key chunks, npiece of them, one
  // workgroup per (query block, head, piece) writing partial results to
  // ws_split ([npiece][B * H * Sq] records of 4 floats, or of D for dQ), which
  // a merge kernel combines in piece order.
  float *ws_split;
  int npiece, piece_chunks;
};

__device__ __forceinline__ int kr(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

template <typename T> struct MT;

template <> struct MT<bf16> {
  static constexpr int KS = 16;
  static constexpr int KL = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Steps needed to contract the 32 rows of one C tile.
  static constexpr int CSTEPS = 2;
};

template <> struct MT<float> {
  static constexpr int KS = 2;
  static constexpr int KL = 1;
  typedef float frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static constexpr int CSTEPS = 16;
};

// KL consecutive elements of a row starting at column d0 (global memory).
template <typename T>
__device__ __forceinline__ typename MT<T>::frag load_frag(const T *row, int d0, bool valid);
template <>
__device__ __forceinline__ bf16x8 load_frag<bf16>(const bf16 *row, int d0, bool valid) {
  return valid ? *reinterpret_cast<const bf16x8 *>(row + d0) : bf16x8{};
}
template <>
__device__ __forceinline__ float load_frag<float>(const float *row, int d0, bool valid) {
  return valid ? row[d0] : 0.f;
}

// A fragment with every element negated: the sign bits flipped, one 32-bit
// xor per register (exact).
template <typename T>
__device__ __forceinline__ typename MT<T>::frag neg_frag(typename MT<T>::frag f);
template <> __device__ __forceinline__ bf16x8 neg_frag<bf16>(bf16x8 f) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, f) ^ 0x80008000u);
}
template <> __device__ __forceinline__ float neg_frag<float>(float f) { return -f; }

// Dot product of two fragments (a lane's KL elements), fp32.
template <typename T>
__device__ __forceinline__ float frag_dot(typename MT<T>::frag a, typename MT<T>::frag b);
template <> __device__ __forceinline__ float frag_dot<bf16>(bf16x8 a, bf16x8 b) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = fmaf((float)a[e], (float)b[e], s);
  return s;
}
template <> __device__ __forceinline__ float frag_dot<float>(float a, float b) { return a * b; }

// Pack C-tile values as a C-reuse B operand for step `st` (see header).
template <typename T>
__device__ __forceinline__ typename MT<T>::frag creuse(const float *v, int st);
template <>
__device__ __forceinline__ bf16x8 creuse<bf16>(const float *v, int st) {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (bf16)v[8 * st + e];
  return f;
}
template <>
__device__ __forceinline__ float creuse<float>(const float *v, int st) {
  return v[st];
}

// ---------------------------------------------------------------------------
// LDS tile holding one 32- or 64-row chunk of a strided [S, D] matrix.
//
// bf16: rows are laid out in groups of four, row r at byte offset
// (r / 4) * G + (r % 4) * RS.  gfx950 LDS has 64 banks of 4 bytes; it serves a
// ds_read_b128 16 lanes at a time and a ds_read_b64_tr_b16 32 lanes at a time.
// The A-operand read (16 consecutive rows, same 16 bytes) is conflict-free iff
// those rows start at 16 distinct multiples of 16 modulo 256; the C-reuse read
// (4 consecutive rows of one group, 64 bytes each) iff the 4 rows start in 4
// different 64-byte quarters modulo 256.  RS = 64 (mod 256) for D = 32,
// 192 or 320 for D = 64 / 128 spreads a group's rows over the quarters, and
// G = 16 (mod 64) shifts successive groups by 16 bytes: both patterns are
// conflict-free, and each fragment read of a lane is one base address plus a
// compile-time offset.  The tile is filled by direct global -> LDS loads that
// write whole 1 KB segments (see ChunkIO), so it is sized in segments, a
// multiple of 4 of them so that every wave issues the same number of loads.
//
// fp32: rows of D + 1 floats; 32 lanes reading one column of 32 rows hit 32
// different banks.
template <typename T, int D, int ROWS = 32> struct Tile;

// Row stride in 16-byte slots: the smallest >= D / 8 that is 4 or 12 mod 16
// (a group's 4 rows then fall in 4 different quarters); group stride: the
// smallest odd slot count that holds the group (odd: successive groups shift by
// one 16-byte slot mod 4).  D = 32 / 64 / 128 give 32 / 96 / 160 and
// 136 / 360 / 616 elements.
constexpr int tile_rs_slots(int d8) { return (d8 % 16 == 4 || d8 % 16 == 12) ? d8 : tile_rs_slots(d8 + 1); }
constexpr int tile_g_slots(int need) { return need % 2 ? need : need + 1; }

template <int D, int ROWS> struct Tile<bf16, D, ROWS> {
  static_assert(D % 32 == 0, "tile width");
  static constexpr int RS = 8 * tile_rs_slots(D / 8);               // row stride in a group, elements
  static constexpr int G = 8 * tile_g_slots((3 * RS + D) / 8);      // group stride, elements
  static constexpr int SLOTS = ROWS / 4 * G / 8;                     // 16-byte slots of all groups
  static constexpr int NSEG = ((SLOTS + 63) / 64 + 3) / 4 * 4;       // 1 KB load segments
  bf16 a[NSEG * 512];
  __device__ __forceinline__ static constexpr int row_off(int r) { return (r >> 2) * G + (r & 3) * RS; }
  // A operand of a contraction over columns: row r, step s.
  __device__ __forceinline__ bf16x8 frag(int r, int s, int half) const {
    return *reinterpret_cast<const bf16x8 *>(&a[row_off(r) + 16 * s + 8 * half]);
  }
  // A operand of a C-reuse product: column n0 + (lane's n), rows
  // r0 + kidx(st, half, e) (r0 a multiple of 32).
  // ds_read_b64_tr_b16 hands lane i of each 16-lane group element i % 4 of the
  // 8 bytes addressed by lanes i / 4 + 4 e (e = 0..3); so lane i addresses row
  // rowbase + i / 4, columns colbase + 4 (i % 4) .. + 3, and receives rows
  // rowbase .. rowbase + 3 of column colbase + i.  rowbase = r0 + 16 st +
  // 4 half (+ 8) is a multiple of 4, so the row offset splits into a per-lane
  // part and a compile-time group offset.
  __device__ __forceinline__ bf16x8 tfrag(int n0, int st, int lane, int r0 = 0) const {
    const int i = lane & 15, g = lane >> 4, half = lane >> 5;
    const int base = half * G + (i >> 2) * RS + 16 * (g & 1) + 4 * (i & 3);
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)(const_cast<bf16 *>(&a[base + (r0 / 4 + 4 * st) * G + n0])));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)(const_cast<bf16 *>(&a[base + (r0 / 4 + 4 * st + 2) * G + n0])));
    const bf16x4 l = __builtin_bit_cast(bf16x4, lo), h = __builtin_bit_cast(bf16x4, hi);
    return bf16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
  }
};

template <int D, int ROWS> struct Tile<float, D, ROWS> {
  static constexpr int LD = D + 1;
  float a[ROWS * LD];
  __device__ __forceinline__ void put(int r, int c, f32x4 x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[r * LD + 4 * c + e] = x[e];
  }
  __device__ __forceinline__ float frag(int r, int s, int half) const {
    return a[r * LD + 2 * s + half];
  }
  __device__ __forceinline__ float tfrag(int n0, int st, int lane, int r0 = 0) const {
    return a[(r0 + kr(st, lane >> 5)) * LD + n0 + (lane & 31)];
  }
};

// Direct global -> LDS loads (gfx950 global_load_lds_dword[x4]): every lane of
// the wave reads `bytes` bytes at its own global address and the wave writes
// them to LDS at lds + bytes * lane.  Issued as inline assembly on purpose: the
// compiler then does not track them, so it neither waits for all of them at
// every barrier nor before LDS reads it cannot prove independent of them.  The
// kernels wait for exactly the loads they need with wait_vmem_le<N>() before
// the barrier that publishes the data.  (Loads the compiler does not see can
// only make its own in-order vmcnt waits stricter, never looser.)  No other
// code here uses M0.
__device__ __forceinline__ unsigned lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(__attribute__((address_space(3))) const void *)p);
}
// m0 = LDS byte address (wave-uniform, in an SGPR), g = this lane's global
// address.
__device__ __forceinline__ void dma_lds16_m0(unsigned m0, const void *g) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(g)
               : "memory");
}
__device__ __forceinline__ void dma_lds16(void *lds, const void *g) { dma_lds16_m0(lds_addr(lds), g); }
// The same with a wave-uniform 64-bit base and a 32-bit per-lane byte offset
// (saddr form: no per-lane 64-bit address arithmetic); m0 = LDS byte address.
__device__ __forceinline__ void dma_lds16_at(unsigned m0, const void *sbase, unsigned voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(sbase)
               : "memory");
}
__device__ __forceinline__ void dma_lds4_at(unsigned m0, const void *g) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(m0), "v"(g)
               : "memory");
}
__device__ __forceinline__ void dma_lds4(void *lds, const void *g) { dma_lds4_at(lds_addr(lds), g); }

// s_waitcnt vmcnt(n), other counters unconstrained (n < 64: the count's low
// four bits sit in bits 3:0 of the immediate, its high two in bits 15:14).
template <int N> __device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vmem() { wait_vmem_le<0>(); }

// Streams ROWS-row chunks of a strided [S, D] matrix into a Tile.  issue() starts
// the transfer of rows [r0, r0 + ROWS) (rows past the end repeat the last row, so
// every tile element is finite and no lane branches).  The data must have
// landed, in every wave, before the barrier that hands the tile over: for bf16
// that is a vmcnt wait (LOADS = the number of loads one issue() leaves in
// flight per wave), for fp32 it is complete(), which writes the registers.
//
// bf16: gfx950 direct loads (global_load_lds_dwordx4): one instruction writes
// the 16 bytes of lane i at LDS segment base + 16 i, so each wave fills whole
// 1 KB segments and lane i fetches whichever row chunk belongs at that slot
// (pad slots and the slack past the last row fetch a harmless duplicate).
// No registers or LDS write instructions are involved.
// fp32: a register prefetch written to LDS by complete().
template <typename T, int D, int ROWS = 32> struct ChunkIO;

template <int D, int ROWS> struct ChunkIO<bf16, D, ROWS> {
  typedef Tile<bf16, D, ROWS> TileT;
  static constexpr int LOADS = TileT::NSEG / 4;
  static constexpr bool DIRECT = true;
  unsigned off[LOADS];  // byte offset of load j from the chunk's first row
  int wave;
  // Chunk row and column of this lane's load j (pad slots: row ROWS - 1, col 0).
  __device__ __forceinline__ void slot_rc(int j, int &row, int &col) const {
    const int lane = threadIdx.x & 63;
    const int slot = (wave + 4 * j) * 64 + lane;  // 16-byte slot of the tile
    const int grp = slot / (TileT::G / 8), o = slot % (TileT::G / 8);
    const int q = o / (TileT::RS / 8), c = o % (TileT::RS / 8);
    const bool data = grp < ROWS / 4 && q < 4 && c < D / 8;
    row = data ? 4 * grp + q : ROWS - 1;
    col = data ? 8 * c : 0;
  }
  // stride: elements between consecutive rows of the streamed matrix.
  __device__ __forceinline__ void init(int64_t stride) {
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      int row, col;
      slot_rc(j, row, col);
      off[j] = (unsigned)((row * stride + col) * 2);
    }
  }
  // LDS byte address of load j's segment of tile t.
  __device__ __forceinline__ unsigned seg(const TileT &t, int j) const {
    return lds_addr(t.a) + ((wave + 4 * j) << 10);
  }
  // Rows given by a functor: rowptr(r) is the start of chunk row r (0 <= r < ROWS).
  template <typename F> __device__ __forceinline__ void issue_at(F rowptr, TileT &t) {
    issue_elem([&](int r, int c) { return rowptr(r) + c; }, t);
  }
  // Elements given by a functor: elem(r, c) addresses columns c .. c + 7 of chunk
  // row r (c a multiple of 8), so a row may be assembled from several sources.
  template <typename F> __device__ __forceinline__ void issue_elem(F elem, TileT &t) {
    issue_elem_at(elem, lds_addr(t.a));
  }
  // The same into the tile at LDS byte address tile_lds (see issue_one_at).
  template <typename F> __device__ __forceinline__ void issue_elem_at(F elem, unsigned tile_lds) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      int row, col;
      slot_rc(j, row, col);
      dma_lds16_m0(tile_lds + ((wave + 4 * j) << 10), elem(row, col));
    }
  }
  // Load j alone of issue() below, branch-free (the loads of one chunk may be
  // spread over the previous chunk's compute; see the dK / dV kernel): cb is
  // the chunk's first row, last = nrows - 1 - r0 >= 0, rstride = bytes per row.
  // The offset is capped at that of row `last`'s final 16-byte segment: a lane
  // of a row <= last keeps its own (for any row stride, row * rstride + 2 col
  // stays at or below that bound), a lane past the end reads that segment
  // (finite data of the matrix, which the mask keeps out of every result).
  // One unsigned min per load; the bound is wave-uniform.
  __device__ __forceinline__ void issue_one(int j, const bf16 *cb, int last, unsigned rstride,
                                            TileT &t) {
    issue_one_at(j, cb, last, rstride, lds_addr(t.a));
  }
  // The same with the tile given by its LDS byte address (a wave-uniform
  // integer: a tile picked at run time then costs no generic-pointer
  // arithmetic).
  __device__ __forceinline__ void issue_one_at(int j, const bf16 *cb, int last, unsigned rstride,
                                               unsigned tile_lds) {
    const unsigned cap = (unsigned)min(last, ROWS - 1) * rstride + 2u * (D - 8);
    dma_lds16_at(tile_lds + ((wave + 4 * j) << 10), cb, min(off[j], cap));
  }
  // Rows [r0, r0 + ROWS) of a matrix with `stride` (the one given to init) and
  // `nrows` rows; rows past the end repeat the last row.  r0 < nrows.
  __device__ __forceinline__ void issue(const bf16 *base, int64_t stride, int r0, int nrows,
                                        TileT &t) {
    const bf16 *cb = base + (int64_t)r0 * stride;  // wave-uniform
    if (r0 + ROWS <= nrows) {
#pragma unroll
      for (int j = 0; j < LOADS; ++j) dma_lds16_at(seg(t, j), cb, off[j]);
    } else {
      const int last = nrows - 1 - r0;
#pragma unroll
      for (int j = 0; j < LOADS; ++j) {
        int row, col;
        slot_rc(j, row, col);
        dma_lds16_at(seg(t, j), cb, (unsigned)((min(row, last) * stride + col) * 2));
      }
    }
  }
  __device__ __forceinline__ void complete(TileT &) {}
};

template <int D, int ROWS> struct ChunkIO<float, D, ROWS> {
  typedef Tile<float, D, ROWS> TileT;
  static constexpr int LOADS = 0;
  static constexpr bool DIRECT = false;
  static constexpr int CH = D / 4;  // 16-byte chunks per row
  static constexpr int PER = (ROWS * CH + 255) / 256;
  f32x4 r[PER];
  __device__ __forceinline__ void init(int64_t) {}
  template <typename F> __device__ __forceinline__ void issue_at(F rowptr, TileT &t) {
    issue_elem([&](int row, int c) { return rowptr(row) + c; }, t);
  }
  // elem(r, c): columns c .. c + 3 of chunk row r (c a multiple of 4).
  template <typename F> __device__ __forceinline__ void issue_elem(F elem, TileT &) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int id = threadIdx.x + 256 * j;
      r[j] = (ROWS * CH % 256 == 0 || id < ROWS * CH)
                 ? *reinterpret_cast<const f32x4 *>(elem(id / CH, 4 * (id % CH)))
                 : f32x4{};
    }
  }
  __device__ __forceinline__ void issue(const float *base, int64_t stride, int r0, int nrows,
                                        TileT &t) {
    issue_at([&](int r) { return base + (int64_t)min(r0 + r, nrows - 1) * stride; }, t);
  }
  __device__ __forceinline__ void complete(TileT &t) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int id = threadIdx.x + 256 * j;
      if (ROWS * CH % 256 == 0 || id < ROWS * CH) t.put(id / CH, id % CH, r[j]);
    }
  }
};

// Visibility of (query i, key j) by the index rule.
__device__ __forceinline__ bool idx_visible(const DenseParams &p, int i, int j) {
  const int d = j - i;
  return i < p.Sq && j < p.Sk && d >= p.lo_off && d <= p.hi_off;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum / max of x over lanes i and i ^ 32 (the two halves of the wave), through
// v_permlane32_swap: a VALU exchange, no LDS round trip.  The swap returns
// (lanes 0-31 of x in both halves, lanes 32-63 of x in both halves); both
// operations are commutative, so every lane gets the bits of
// op(x, x of lane ^ 32).
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// x, made opaque to the optimiser: what is derived from it is computed where it
// is used instead of being hoisted out of a loop and kept live across it (in a
// register the loop body needs, or in scratch memory).
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Computes x here: an empty asm that reads and rewrites it, so the value is
// formed before this point and the optimiser cannot sink its computation into
// a later block (past a branch that follows it), where nothing would hide it.
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(bf16x8 &x) { asm volatile("" : "+v"(x)); }


// Workgroup id -> logical tile id.  The hardware hands workgroup i to XCD i % 8;
// this gives every XCD a contiguous range of logical ids, so the tiles of one
// (b, h) head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = bid & 7, idx = bid >> 3;
  return x * per + (x < rem ? x : rem) + idx;
}

// Workgroup id -> (head, rank) for a grid of n = heads * nb tiles, nb per head
// (tile_of_logical: the same for the logical id L = xcd_remap(id, n)).
// Every XCD gets a contiguous range of heads (their tiles share its L2).  When
// the heads split evenly over the 8 XCDs, an XCD takes its heads GS at a time
// (all of them if GS does not divide their count) and runs each group's tiles
// rank by rank: rank 0 (the caller's heaviest tile) of the group's heads, then
// rank 1, ...  Workgroups start in id order on each XCD, so long tiles start
// early and short ones fill in at the end (close to greedy longest-first),
// while only about GS heads' operands are in flight in the XCD's L2 at a time.
// Otherwise the order is head by head.
template <int GS>
__device__ __forceinline__ void tile_of_logical(int L, int n, int nb, int &head, int &rank) {
  if (n % (8 * nb) == 0) {
    const int hp = n / (8 * nb);  // heads per XCD
    const int gs = hp % GS == 0 ? GS : hp;
    const int x = L / (hp * nb), idx = L % (hp * nb);
    const int grp = idx / (gs * nb), w = idx % (gs * nb);
    rank = w / gs;
    head = x * hp + grp * gs + w % gs;
  } else {
    head = L / nb;
    rank = L % nb;
  }
}
template <int GS>
__device__ __forceinline__ void tile_order(int bid, int n, int nb, int &head, int &rank) {
  tile_of_logical<GS>(xcd_remap(bid, n), n, nb, head, rank);
}

// A narrow band: a window rule whose visible span (hi_off - lo_off + 1 index
// differences) is at most a quarter of the shorter sequence.  Then every block
// but the few at the band's clipped end sees the same number of chunks, and
// the heavy-first order starts every CU on an equal block: all of them load
// their first operands and store their results at the same moments, round
// after round.  Starting with the short end blocks puts part of each XCD's
// CUs ahead of the rest for the whole kernel (the total work is unchanged).
__device__ __forceinline__ bool narrow_band(const DenseParams &p) {
  return p.lo_off > -kBig && 4 * ((int64_t)p.hi_off - p.lo_off + 1) <= (int64_t)min(p.Sq, p.Sk);
}

// Store 4 consecutive fp32 values as T.
template <typename T> __device__ __forceinline__ void store4(T *dst, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<bf16>(bf16 *dst, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4 *>(dst) = bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
template <> __device__ __forceinline__ void store4<float>(float *dst, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4 *>(dst) = f32x4{a, b, c, d};
}

// Stores a wave's accumulator tiles acc[D / 32] -- lane column n = l32 is row n
// of the output, tile t's element r is column 32 t + kr(r, half) -- times
// `scale` as rows 0 .. nvalid - 1 of a [32, D] matrix of T whose row n starts
// at rowptr(n).  Straight from the C layout each store instruction would
// scatter 64 small pieces over 32 rows; instead the wave writes the tiles to
// `lds` (its own 32 * (D * sizeof(T) + 16) bytes, 16-byte aligned, free) and
// reads them back row-major, so every lane stores 16 contiguous bytes and
// consecutive lanes fill whole rows.  `scale` may differ per lane (row).  The caller synchronises the wave's LDS
// (a barrier) between writes and reads: write_tiles(), barrier, store_rows().
template <typename T, int D> struct RowStore {
  static constexpr int ES = sizeof(T), RB = D * ES + 16;  // padded row bytes
  static constexpr int BYTES = 32 * RB;
  static constexpr int LPR = D * ES / 16, RPI = 64 / LPR;  // lanes per row, rows per instruction
  // NEG: the tiles hold the negated values; 0 - scale * acc restores them
  // exactly and keeps a zero +0.
  template <bool NEG = false>
  __device__ __forceinline__ static void write_tiles(const f32x16 *acc, float scale, char *lds,
                                                     int lane) {
    const int l32 = lane & 31, half = lane >> 5;
    auto v = [&](int t, int r) { return NEG ? 0.f - scale * acc[t][r] : scale * acc[t][r]; };
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4<T>(reinterpret_cast<T *>(lds + l32 * RB) + 32 * t + 8 * g + 4 * half,
                  v(t, 4 * g), v(t, 4 * g + 1), v(t, 4 * g + 2), v(t, 4 * g + 3));
  }
  template <typename F>
  __device__ __forceinline__ static void store_rows(const char *lds, int nvalid, F rowptr, int lane) {
    const int c = lane % LPR;
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int n = it * RPI + lane / LPR;
      const f32x4 x = *reinterpret_cast<const f32x4 *>(lds + n * RB + 16 * c);
      T *dst = n < nvalid ? rowptr(n) : nullptr;  // rowptr may return nullptr: no such row
      if (dst) *reinterpret_cast<f32x4 *>(reinterpret_cast<char *>(dst) + 16 * c) = x;
    }
  }
};

}  // namespace attn
