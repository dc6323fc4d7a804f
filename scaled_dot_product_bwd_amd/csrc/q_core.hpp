// q_core.hpp -- pieces shared by the query-major kernels (row statistics, dQ,
// statistics + dQ).
//
// A wave owns NQB blocks of 32 queries (one query per lane column l32 in each
// block); their Q and dY rows sit in registers as MFMA B operands.  Keys stream
// through LDS in chunks of 32 (64 in the fused statistics + dQ pass).  Phase A of a chunk forms, per query block,
//   S^T = K Q^T and dP^T = V dY^T     (rows = the chunk's keys, A from LDS)
// as C tiles whose element r of a lane is key kr(r, half) of the chunk for the
// lane's query.  Every K / V fragment is read from LDS once and used for all
// NQB query blocks (two for bf16), so each 1 KB LDS read feeds NQB MFMAs.
#pragma once

#include "device_common.hpp"
#include "kv_core.hpp"

namespace attn {

template <typename T> struct QShape {
  static constexpr int NQB = 1;  // 32-query blocks per wave
  static constexpr int QROWS = 4 * 32 * NQB;           // queries per workgroup
};

// Phase A for every query block.  The K / V fragments of k-step s are read
// three steps ahead (a ring of four) and feed the MFMAs of all query blocks.
// dma(s), s < NDMA: the caller's s-th direct-to-LDS load for a later chunk,
// one per step, so a wave's stall on a busy vector-memory pipe falls under
// its running MFMAs (as in the dK / dV body).
// RING: fragment registers per operand (reads run RING - 1 steps ahead).
template <typename T, int D, int NQB, int NDMA = 0, typename Dma = NoDma, int RING = 4>
__device__ __forceinline__ void q_phase_a(const Tile<T, D> *Kc, const Tile<T, D> *Vc,
                                          const typename MT<T>::frag (*qf)[D / MT<T>::KS],
                                          const typename MT<T>::frag (*gf)[D / MT<T>::KS],
                                          f32x16 *sacc, f32x16 *pacc, int lane, Dma dma = Dma()) {
  typedef MT<T> M;
  constexpr int NSD = D / M::KS;
  const int l32 = lane & 31, half = lane >> 5;
  typename M::frag ka[RING], va[RING];
  auto load = [&](int s) {
    ka[s % RING] = Kc->frag(l32, s, half);
    va[s % RING] = Vc->frag(l32, s, half);
  };
#pragma unroll
  for (int s = 0; s < RING - 1 && s < NSD; ++s) load(s);
#pragma unroll
  for (int q = 0; q < NQB; ++q) sacc[q] = pacc[q] = f32x16{};
  static_assert(NDMA <= NSD, "one load per step");
#pragma unroll
  for (int s = 0; s < NSD; ++s) {
    if (s + RING - 1 < NSD) load(s + RING - 1);
    if (s < NDMA) dma(s);
#pragma unroll
    for (int q = 0; q < NQB; ++q) {
      sacc[q] = M::mma(ka[s % RING], qf[q][s], sacc[q]);
      pacc[q] = M::mma(va[s % RING], gf[q][s], pacc[q]);
    }
  }
}

// Query-major chunk ranges of a workgroup holding queries [i0, i0 + QROWS),
// in chunks of KC keys: the visible chunks [c_first, c_last] and, inside them,
// the chunks [cu0, cu1] whose every (query, key) pair the index rule keeps (no
// per-element test).
struct QRange {
  int c_first, c_last, cu0, cu1;
};
template <int KC = 32>
__device__ __forceinline__ QRange q_range(const DenseParams &p, int i0, int qrows, bool index_only) {
  static_assert(KC == 32 || KC == 64, "chunk size");
  constexpr int SH = KC == 32 ? 5 : 6;
  QRange r;
  const int ilast = min(i0 + qrows, p.Sq) - 1;
  const int jlo = max(0, (int)max((int64_t)i0 + p.lo_off, (int64_t)0));
  const int jhi = min(p.Sk - 1, (int)min((int64_t)ilast + p.hi_off, (int64_t)kBig));
  r.c_first = jlo >> SH;
  r.c_last = jhi >= jlo ? jhi >> SH : r.c_first - 1;
  r.cu0 = r.c_last + 1;
  r.cu1 = r.c_last;
  if (index_only && i0 + qrows <= p.Sq) {
    // key j of chunk c: j0 + KC - 1 - i0 <= hi_off, j0 - (i0 + qrows - 1) >= lo_off, j0 + KC <= Sk
    const int64_t c_hi = min(((int64_t)i0 + p.hi_off - (KC - 1)) >> SH, (int64_t)(p.Sk >> SH) - 1);
    const int64_t lo_j = (int64_t)i0 + qrows - 1 + p.lo_off;
    const int64_t c_lo = lo_j <= 0 ? 0 : (lo_j + KC - 1) >> SH;
    int64_t a = max(c_lo, (int64_t)r.c_first), b = min(c_hi, (int64_t)r.c_last);
    if (a <= b) {
      r.cu0 = (int)a;
      r.cu1 = (int)b;
    }
  }
  return r;
}

}  // namespace attn

namespace attn {

// Online row statistics, log2 domain, with a lazily moved reference.
// Per query row (a lane column; the wave's two halves hold different keys of
// the same row): l = sum 2^(s - mref) and dl = sum 2^(s - mref) dP over the
// keys seen so far, where the reference mref moves to a chunk's max only when
// that max exceeds it by more than kRefSlack.  The terms 2^(s - mref) then
// stay <= 2^kRefSlack, and after the first visible chunk almost no chunk
// rescales anything (a caller that carries accumulators in the same scale
// multiplies them only then).  mtrue is the running max itself.  The row
// statistics kernel (32-key chunks) and the fused statistics + dQ kernel
// (64-key chunks, the same stages) both use this arithmetic.
constexpr float kRefSlack = 8.f;

struct RowStat {
  float mref, mtrue, l, dl;
  __device__ __forceinline__ void init() {
    mref = mtrue = -INFINITY;
    l = dl = 0.f;
  }
};

// The reference update for a chunk whose (both halves') max score is mx.
__device__ __forceinline__ float row_stat_ref(RowStat &st, float mx, bool &moved, float &mu) {
  st.mtrue = fmaxf(st.mtrue, mx);
  moved = mx > st.mref + kRefSlack;  // false while every key so far is hidden
  const float al = moved ? fast_exp2(st.mref - mx) : 1.f;  // 0 from mref = -inf
  if (moved) st.mref = mx;
  mu = st.mref == -INFINITY ? 0.f : st.mref;
  return al;
}

// The sums: l = l al + sum pr, dl = dl al + sum pr dP.
__device__ __forceinline__ void row_stat_sum(RowStat &st, const float *pr, const f32x16 &pacc,
                                             float al) {
  float ls = 0.f, ds = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    ls += pr[r];
    ds = fmaf(pr[r], pacc[r], ds);
  }
  st.l = fmaf(st.l, al, ls);
  st.dl = fmaf(st.dl, al, ds);
}

// One 32-key chunk into the statistics.  sacc[r]: the raw score accumulator
// (Q . K) of the lane's key r, pacc[r] its dP, c = scale log2 e.  Writes
// pr[r] = 2^(s2[r] - mref), s2 = sacc c + adj(r) the log2-domain score, and
// returns the factor by which earlier terms were rescaled (1 if mref did not
// move); `moved` tells whether it did, for this lane's row.  `plain` (a chunk
// every key of which is visible, no bias, c > 0) skips the mask term, takes
// the max on the raw accumulators (max(x) c == max(x c) exactly for c > 0)
// and folds c into the exponent's FMA.
template <typename Adj>
__device__ __forceinline__ float row_stat_chunk(RowStat &st, const f32x16 &sacc,
                                                const f32x16 &pacc, float c, bool plain, Adj adj,
                                                float *pr, bool &moved) {
  float mu, al;
  if (plain) {
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = halves_max(mx) * c;
    al = row_stat_ref(st, mx, moved, mu);
#pragma unroll
    for (int r = 0; r < 16; ++r) pr[r] = fast_exp2(fmaf(sacc[r], c, -mu));
  } else {
    float s2[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) s2[r] = fmaf(sacc[r], c, adj(r));
    float mx = s2[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s2[r]);
    mx = halves_max(mx);
    al = row_stat_ref(st, mx, moved, mu);
#pragma unroll
    for (int r = 0; r < 16; ++r) pr[r] = fast_exp2(s2[r] - mu);
  }
  row_stat_sum(st, pr, pacc, al);
  return al;
}

// Final statistics of a row into the workspace planes (both halves call it;
// the caller lets one store).  l_tot / dl_tot: the two halves' sums combined.
struct RowStatOut {
  float m, l, delta, nls, inv_l;
  bool empty;
};
__device__ __forceinline__ RowStatOut row_stat_final(const RowStat &st, float inv_scale_log2) {
  RowStatOut o;
  const float l_tot = halves_sum(st.l);
  const float d_tot = halves_sum(st.dl);
  o.empty = !(l_tot > 0.f);
  o.m = o.empty ? -INFINITY : st.mtrue * kLn2;
  o.l = o.empty ? 0.f : l_tot * fast_exp2(st.mref - st.mtrue);
  o.delta = o.empty ? 0.f : d_tot / l_tot;
  o.nls = (o.empty ? -INFINITY : -(st.mref + __log2f(l_tot))) * inv_scale_log2;
  o.inv_l = o.empty ? 0.f : 1.f / l_tot;
  return o;
}

}  // namespace attn
