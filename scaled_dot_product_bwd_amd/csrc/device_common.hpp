// device_common.hpp -- shared device helpers for the gfx950 attention-backward
// kernels: element types, 32x32 MFMA wrappers, fragment layouts, LDS tiles,
// mask evaluation and the workgroup -> tile mapping.
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
// r the lane stands for row kr(r, half).  The matching A operand reads the same
// rows from LDS.  No register shuffles are needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
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
  __device__ __forceinline__ static frag zero() { return frag{}; }
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
  __device__ __forceinline__ static frag zero() { return 0.f; }
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
// LDS tiles of ROWS rows x D columns.
//
// RowTile: row-major, padded so that the A-operand reads (32 lanes on 32 rows,
// same columns) spread over all banks: +8 bf16 (16 B) or +1 float per row.
// TTile (bf16 only): the same data transposed, [D][ROWS + 4], for the A operand
// of a C-reuse product, which needs 4 consecutive rows of one column.
template <typename T, int ROWS, int D> struct RowTile;

template <int ROWS, int D> struct RowTile<bf16, ROWS, D> {
  static constexpr int LD = D + 8;
  bf16 a[ROWS * LD];
  // A operand of a contraction over columns: row `row`, step s.
  __device__ __forceinline__ bf16x8 frag(int row, int s, int half) const {
    return *reinterpret_cast<const bf16x8 *>(&a[row * LD + s * 16 + half * 8]);
  }
  __device__ __forceinline__ void put8(int row, int c0, bf16x8 x) {
    *reinterpret_cast<bf16x8 *>(&a[row * LD + c0]) = x;
  }
};

template <int ROWS, int D> struct RowTile<float, ROWS, D> {
  static constexpr int LD = D + 1;
  float a[ROWS * LD];
  __device__ __forceinline__ float frag(int row, int s, int half) const {
    return a[row * LD + 2 * s + half];
  }
  __device__ __forceinline__ float at(int row, int col) const { return a[row * LD + col]; }
  __device__ __forceinline__ void put4(int row, int c0, f32x4 x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a[row * LD + c0 + e] = x[e];
  }
};

template <int ROWS, int D> struct TTile {
  static constexpr int LD = ROWS + 4;
  bf16 a[D * LD];
  // A operand of a C-reuse product for column n, step s (rows kidx(s, half, e)).
  __device__ __forceinline__ bf16x8 frag(int n, int s, int half) const {
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(&a[n * LD + 16 * s + 4 * half]);
    const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(&a[n * LD + 16 * s + 8 + 4 * half]);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ __forceinline__ void put8(int row, int c0, bf16x8 x) {
#pragma unroll
    for (int e = 0; e < 8; ++e) a[(c0 + e) * LD + row] = x[e];
  }
};

// A operand of a C-reuse product (column n, step st) from the LDS copy of the
// contracted rows: the transposed tile for bf16, the row-major tile for fp32.
template <typename T, int ROWS, int D> struct CReuseSrc;
template <int ROWS, int D> struct CReuseSrc<bf16, ROWS, D> {
  typedef TTile<ROWS, D> tile;
  __device__ __forceinline__ static bf16x8 frag(const tile &t, int n, int st, int half) {
    return t.frag(n, st, half);
  }
};
template <int ROWS, int D> struct CReuseSrc<float, ROWS, D> {
  typedef RowTile<float, ROWS, D> tile;
  __device__ __forceinline__ static float frag(const tile &t, int n, int st, int half) {
    return t.at(kr(st, half), n);
  }
};

// Stage 32 rows [r0, r0 + 32) of a strided [S, D] matrix into LDS, row-major and
// (bf16, if `tt` is given) transposed.  Rows >= nrows are zero.  Thread t moves
// 16 bytes of row t % 32 per pass, so each pass writes 32 different rows.
template <typename T, int D>
__device__ __forceinline__ void stage_rows(const T *base, int64_t row_stride, int r0, int nrows,
                                           RowTile<T, 32, D> &rt, TTile<32, D> *tt = nullptr) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int CH = D / VEC;  // 16-byte chunks per row
  const int t = threadIdx.x;
  const int row = t & 31;
  const bool valid = r0 + row < nrows;
  const T *src = base + (int64_t)(valid ? r0 + row : 0) * row_stride;
#pragma unroll
  for (int c = t >> 5; c < CH; c += 8) {
    if constexpr (sizeof(T) == 2) {
      const bf16x8 x = valid ? *reinterpret_cast<const bf16x8 *>(src + c * VEC) : bf16x8{};
      rt.put8(row, c * VEC, x);
      if (tt) tt->put8(row, c * VEC, x);
    } else {
      const f32x4 x = valid ? *reinterpret_cast<const f32x4 *>(src + c * VEC) : f32x4{};
      rt.put4(row, c * VEC, x);
    }
  }
}

// Stage 32 rows [r0, r0 + 32) of a strided bf16 [S, D] matrix into LDS
// transposed only.
template <int D>
__device__ __forceinline__ void stage_cols(const bf16 *base, int64_t row_stride, int r0, int nrows,
                                           TTile<32, D> &tt) {
  constexpr int VEC = 8, CH = D / VEC;
  const int t = threadIdx.x;
  const int row = t & 31;
  const bool valid = r0 + row < nrows;
  const bf16 *src = base + (int64_t)(valid ? r0 + row : 0) * row_stride;
#pragma unroll
  for (int c = t >> 5; c < CH; c += 8) {
    const bf16x8 x = valid ? *reinterpret_cast<const bf16x8 *>(src + c * VEC) : bf16x8{};
    tt.put8(row, c * VEC, x);
  }
}

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

// log2-domain score of (i, j) from the raw dot product, with the mask applied:
// -inf when hidden.  MODE_INDEX callers skip the per-element test on tiles that
// are entirely visible.
template <int MODE>
__device__ __forceinline__ float masked_score(const DenseParams &p, float dot, int b, int h,
                                              int i, int j, bool check) {
  float s = dot * p.scale_log2;
  if constexpr (MODE == MODE_INDEX) {
    if (check && !idx_visible(p, i, j)) s = -INFINITY;
  } else {
    if (!idx_visible(p, i, j)) {
      s = -INFINITY;
    } else {
      const float mv = p.mask[b * p.ms[0] + h * p.ms[1] + (int64_t)i * p.ms[2] + (int64_t)j * p.ms[3]];
      if constexpr (MODE == MODE_KEYPAD) {
        if (mv < p.thr) s = -INFINITY;
      } else {
        s = fmaf(mv, kLog2e, s);
      }
    }
  }
  return s;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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
