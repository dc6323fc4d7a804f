// q_core.hpp -- pieces shared by the query-major kernels (row statistics, dQ).
//
// A wave owns NQB blocks of 32 queries (one query per lane column l32 in each
// block); their Q and dY rows sit in registers as MFMA B operands.  Keys stream
// through LDS in chunks of 32.  Phase A of a chunk forms, per query block,
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
template <typename T, int D, int NQB, int NDMA = 0, typename Dma = NoDma>
__device__ __forceinline__ void q_phase_a(const Tile<T, D> *Kc, const Tile<T, D> *Vc,
                                          const typename MT<T>::frag (*qf)[D / MT<T>::KS],
                                          const typename MT<T>::frag (*gf)[D / MT<T>::KS],
                                          f32x16 *sacc, f32x16 *pacc, int lane, Dma dma = Dma()) {
  typedef MT<T> M;
  constexpr int NSD = D / M::KS, RING = 4;
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

// Query-major chunk ranges of a workgroup holding queries [i0, i0 + QROWS):
// the visible chunks [c_first, c_last] and, inside them, the chunks [cu0, cu1]
// whose every (query, key) pair the index rule keeps (no per-element test).
struct QRange {
  int c_first, c_last, cu0, cu1;
};
__device__ __forceinline__ QRange q_range(const DenseParams &p, int i0, int qrows, bool index_only) {
  QRange r;
  const int ilast = min(i0 + qrows, p.Sq) - 1;
  const int jlo = max(0, (int)max((int64_t)i0 + p.lo_off, (int64_t)0));
  const int jhi = min(p.Sk - 1, (int)min((int64_t)ilast + p.hi_off, (int64_t)kBig));
  r.c_first = jlo >> 5;
  r.c_last = jhi >= jlo ? jhi >> 5 : r.c_first - 1;
  r.cu0 = r.c_last + 1;
  r.cu1 = r.c_last;
  if (index_only && i0 + qrows <= p.Sq) {
    // key j of chunk c: j0 + 31 - i0 <= hi_off, j0 - (i0 + qrows - 1) >= lo_off, j0 + 32 <= Sk
    const int64_t c_hi = min(((int64_t)i0 + p.hi_off - 31) >> 5, (int64_t)(p.Sk >> 5) - 1);
    const int64_t lo_j = (int64_t)i0 + qrows - 1 + p.lo_off;
    const int64_t c_lo = lo_j <= 0 ? 0 : (lo_j + 31) >> 5;
    int64_t a = max(c_lo, (int64_t)r.c_first), b = min(c_hi, (int64_t)r.c_last);
    if (a <= b) {
      r.cu0 = (int)a;
      r.cu1 = (int)b;
    }
  }
  return r;
}

}  // namespace attn
