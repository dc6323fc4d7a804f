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
  int B, H, Sq, Sk;
  // Index rule: key j is visible to query i iff lo_off <= j - i <= hi_off
  // (and i < Sq, j < Sk).  Causal: hi_off = max(Sk - Sq, 0); window:
  // lo_off = hi_off - w; otherwise +-kBig.
  int lo_off, hi_off;
  int need_dk, need_dv;
  int nblk;  // tiles along the blocked sequence axis
  float *st_m, *st_l, *st_delta, *st_lse2;  // [B * H * Sq] each
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
// LDS tile holding one 32-row chunk of a strided [S, D] matrix, row-major and
// padded, so every fragment read of a lane is one base address plus a
// compile-time offset.
//
// bf16: rows of D + 8 elements (D * 2 + 16 bytes).  The 16-byte pad shifts
// consecutive rows by 4 banks, so the A-operand reads (8 rows x 16 bytes, same
// columns) touch every bank once.  The tile is filled by direct global -> LDS
// loads that write 1 KB segments linearly (see DirectLoader), so it is sized in
// whole segments.
//
// fp32: rows of D + 1 floats; 32 lanes reading one column of 32 rows hit 32
// different banks.
template <typename T, int D> struct Tile;

template <int D> struct Tile<bf16, D> {
  static constexpr int LD = D + 8;                    // row stride, elements
  static constexpr int CPR = LD / 8;                  // 16-byte slots per row (last = pad)
  static constexpr int CH = D / 8;                    // 16-byte data chunks per row
  static constexpr int NSEG = (32 * CPR + 63) / 64;   // 1 KB segments covering 32 rows
  bf16 a[NSEG * 512];
  // A operand of a contraction over columns: row r, step s.
  __device__ __forceinline__ bf16x8 frag(int r, int s, int half) const {
    return *reinterpret_cast<const bf16x8 *>(&a[r * LD + 16 * s + 8 * half]);
  }
  // A operand of a C-reuse product: column n0 + (lane's n), rows kidx(st, half, e).
  // ds_read_b64_tr_b16 hands lane i of each 16-lane group element i % 4 of the
  // 8 bytes addressed by lanes i / 4 + 4 e (e = 0..3); so lane i addresses row
  // rowbase + i / 4, columns colbase + 4 (i % 4) .. + 3, and receives rows
  // rowbase .. rowbase + 3 of column colbase + i.
  __device__ __forceinline__ bf16x8 tfrag(int n0, int st, int lane) const {
    const int i = lane & 15, g = lane >> 4, half = lane >> 5;
    const int base = (4 * half + (i >> 2)) * LD + 16 * (g & 1) + 4 * (i & 3);
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)(const_cast<bf16 *>(&a[base + 16 * st * LD + n0])));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)(const_cast<bf16 *>(&a[base + (16 * st + 8) * LD + n0])));
    const bf16x4 l = __builtin_bit_cast(bf16x4, lo), h = __builtin_bit_cast(bf16x4, hi);
    return bf16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
  }
};

template <int D> struct Tile<float, D> {
  static constexpr int LD = D + 1;
  float a[32 * LD];
  __device__ __forceinline__ void put(int r, int c, f32x4 x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[r * LD + 4 * c + e] = x[e];
  }
  __device__ __forceinline__ float frag(int r, int s, int half) const {
    return a[r * LD + 2 * s + half];
  }
  __device__ __forceinline__ float tfrag(int n0, int st, int lane) const {
    return a[kr(st, lane >> 5) * LD + n0 + (lane & 31)];
  }
};

// Wait until this wave's outstanding global loads (and direct-to-LDS writes)
// have landed: s_waitcnt vmcnt(0), other counters unconstrained.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Streams 32-row chunks of a strided [S, D] matrix into a Tile.  issue() starts
// the transfer of rows [r0, r0 + 32) (rows past the end repeat the last row, so
// every tile element is finite and no lane branches); complete() must run
// before the barrier that hands the tile to the other waves.
//
// bf16: gfx950 direct loads (global_load_lds_dwordx4): one instruction writes
// the 16 bytes of lane i at LDS segment base + 16 i, so each wave fills whole
// 1 KB segments and lane i fetches whichever row chunk belongs at that slot
// (pad slots fetch a harmless duplicate).  No registers or LDS writes involved.
// fp32: a register prefetch written to LDS in complete().
template <typename T, int D> struct ChunkIO;

template <int D> struct ChunkIO<bf16, D> {
  typedef Tile<bf16, D> TileT;
  static constexpr int MAXJ = (TileT::NSEG + 3) / 4;
  int rloc[MAXJ], col[MAXJ];
  int wave;
  __device__ __forceinline__ void init() {
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int g = (wave + 4 * j) * 64 + lane;
      int r = g / TileT::CPR, c = g % TileT::CPR;
      if (c >= TileT::CH) c = 0;
      if (r > 31) r = 31;
      rloc[j] = r;
      col[j] = 8 * c;
    }
  }
  __device__ __forceinline__ void issue(const bf16 *base, int64_t stride, int r0, int nrows,
                                        TileT &t) {
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int seg = wave + 4 * j;
      if (seg < TileT::NSEG) {
        const int row = min(r0 + rloc[j], nrows - 1);
        const bf16 *src = base + (int64_t)row * stride + col[j];
        __builtin_amdgcn_global_load_lds(
            (const void *)src, (__attribute__((address_space(3))) void *)(&t.a[seg * 512]), 16, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void complete(TileT &) { wait_vmem(); }
};

template <int D> struct ChunkIO<float, D> {
  typedef Tile<float, D> TileT;
  static constexpr int CH = D / 4;  // 16-byte chunks per row
  static constexpr int PER = (32 * CH + 255) / 256;
  f32x4 r[PER];
  __device__ __forceinline__ void init() {}
  __device__ __forceinline__ void issue(const float *base, int64_t stride, int r0, int nrows,
                                        TileT &) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int id = threadIdx.x + 256 * j;
      const int row = min(r0 + id / CH, nrows - 1), c = id % CH;
      r[j] = (32 * CH % 256 == 0 || id < 32 * CH)
                 ? *reinterpret_cast<const f32x4 *>(base + (int64_t)row * stride + 4 * c)
                 : f32x4{};
    }
  }
  __device__ __forceinline__ void complete(TileT &t) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int id = threadIdx.x + 256 * j;
      if (32 * CH % 256 == 0 || id < 32 * CH) t.put(id / CH, id % CH, r[j]);
    }
  }
};

// Visibility of (query i, key j) by the index rule.
__device__ __forceinline__ bool idx_visible(const DenseParams &p, int i, int j) {
  const int d = j - i;
  return i < p.Sq && j < p.Sk && d >= p.lo_off && d <= p.hi_off;
}

// True iff every (i, j) of the tile [i0, i0 + 32) x [j0, j0 + 32) is visible by
// the index rule (no per-element test needed in MODE_INDEX).
__device__ __forceinline__ bool tile_all_visible(const DenseParams &p, int i0, int j0) {
  return i0 + 32 <= p.Sq && j0 + 32 <= p.Sk && (j0 + 31) - i0 <= p.hi_off &&
         j0 - (i0 + 31) >= p.lo_off;
}

// True iff no (i, j) of the tile is visible by the index rule.
__device__ __forceinline__ bool tile_none_visible(const DenseParams &p, int i0, int j0) {
  return i0 >= p.Sq || j0 >= p.Sk || j0 - (i0 + 31) > p.hi_off || (j0 + 31) - i0 < p.lo_off;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Turn the 16 raw dot products of a C tile into masked log2-domain scores.
// Element r sits at (query qi(r), key kj(r)) as given by the functors.  The
// index rule is only evaluated on tiles that need it (`check`, wave-uniform),
// and then without branches.
template <int MODE, typename QI, typename KJ>
__device__ __forceinline__ void scores16(const DenseParams &p, const f32x16 &acc, float *s2, int b,
                                         int h, bool check, QI qi, KJ kj) {
#pragma unroll
  for (int r = 0; r < 16; ++r) s2[r] = acc[r] * p.scale_log2;
  if constexpr (MODE == MODE_INDEX) {
    if (check) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s2[r] = idx_visible(p, qi(r), kj(r)) ? s2[r] : -INFINITY;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = qi(r), j = kj(r);
      if (idx_visible(p, i, j)) {
        const float mv = p.mask[b * p.ms[0] + h * p.ms[1] + (int64_t)i * p.ms[2] + (int64_t)j * p.ms[3]];
        if constexpr (MODE == MODE_KEYPAD)
          s2[r] = mv < p.thr ? -INFINITY : s2[r];
        else
          s2[r] = fmaf(mv, kLog2e, s2[r]);
      } else {
        s2[r] = -INFINITY;
      }
    }
  }
}

// Workgroup id -> logical tile id.  The hardware hands workgroup i to XCD i % 8;
// this gives every XCD a contiguous range of logical ids, so the tiles of one
// (b, h) head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = bid & 7, idx = bid >> 3;
  return x * per + (x < rem ? x : rem) + idx;
}

// Store 4 consecutive fp32 values as T.
template <typename T> __device__ __forceinline__ void store4(T *dst, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<bf16>(bf16 *dst, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4 *>(dst) = bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
template <> __device__ __forceinline__ void store4<float>(float *dst, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4 *>(dst) = f32x4{a, b, c, d};
}

}  // namespace attn
