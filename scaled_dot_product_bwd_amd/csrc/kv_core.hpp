// kv_core.hpp -- the per-chunk body shared by the dense and the paged dK / dV
// kernels.
//
// A wave owns 32 keys, one per lane column (l32); their K and V rows sit in
// registers as MFMA B operands, their dK^T and dV^T accumulators as C tiles
// (column = key, rows = head-dim slice of 32).  One call consumes a chunk of
// 32 * NSUB query rows staged in LDS (Q, dY tiles and the row statistics) as
// NSUB independent 32-row sub-tiles, following rlx-cpu 0.2.17
// src/attention_bwd.rs `backward_dense_head_all`:
//   S = Q K^T, dP = dY V^T               rows = queries, A from LDS
//   P = exp2(S * scale * log2 e - lse2)   lse2 = m log2 e + log2 l, per row
//   dS = P (dP - delta) scale
//   dV^T += dY^T P,  dK^T += Q^T dS       A read transposed from LDS, B = C reuse
// The masking of the raw scores is the caller's (`scores`), so the same body
// serves index / padding / bias masks (dense) and page-table token positions
// (paged).
#pragma once

#include "device_common.hpp"

namespace attn {

// Sub-tiles per chunk: two for bf16 (their MFMA / VALU chains interleave within
// the wave and share one barrier); one for fp32, whose tiles are 8x larger per
// row in MFMA steps.
template <typename T> struct KvShape {
  static constexpr int NSUB = sizeof(T) == 2 ? 2 : 1;
  static constexpr int ROWS = 32 * NSUB;
};

// scores(u, acc, sc): turn the raw Q.K dot products `acc` of sub-tile u into the
// 16 masked log2-domain scores sc[] of this lane (element r = query row
// 32 u + kr(r, half) of the chunk, key = this lane's column).
// lse2 / delta: the chunk's per-row statistics in LDS (row i at [i]).
template <typename T, int D, typename Scores>
__device__ __forceinline__ void kv_chunk(const typename MT<T>::frag *kf,
                                         const typename MT<T>::frag *vf, f32x16 *dk, f32x16 *dv,
                                         const Tile<T, D, KvShape<T>::ROWS> *Qc,
                                         const Tile<T, D, KvShape<T>::ROWS> *Gc,
                                         const float *lse2, const float *delta, float scale,
                                         int lane, Scores scores) {
  typedef MT<T> M;
  constexpr int NSD = D / M::KS, NT = D / 32, CS = M::CSTEPS;
  constexpr int NSUB = KvShape<T>::NSUB;
  const int l32 = lane & 31, half = lane >> 5;

  f32x16 sacc[NSUB], pacc[NSUB];
#pragma unroll
  for (int u = 0; u < NSUB; ++u) {
    typename M::frag qa[NSD], ga[NSD];
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      qa[s] = Qc->frag(32 * u + l32, s, half);
      ga[s] = Gc->frag(32 * u + l32, s, half);
    }
    sacc[u] = f32x16{};
    pacc[u] = f32x16{};
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      sacc[u] = M::mma(qa[s], kf[s], sacc[u]);
      pacc[u] = M::mma(ga[s], vf[s], pacc[u]);
    }
  }
  typename M::frag pf[NSUB][CS], sf[NSUB][CS];
#pragma unroll
  for (int u = 0; u < NSUB; ++u) {
    float sc[16], pv[16], dsv[16];
    scores(u, sacc[u], sc);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 lse4 = *reinterpret_cast<const f32x4 *>(&lse2[32 * u + 8 * g + 4 * half]);
      const f32x4 del4 = *reinterpret_cast<const f32x4 *>(&delta[32 * u + 8 * g + 4 * half]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        const float pr = fast_exp2(sc[r] - lse4[e]);
        pv[r] = pr;
        dsv[r] = pr * (pacc[u][r] - del4[e]) * scale;
      }
    }
#pragma unroll
    for (int st = 0; st < CS; ++st) {
      pf[u][st] = creuse<T>(pv, st);
      sf[u][st] = creuse<T>(dsv, st);
    }
  }
#pragma unroll
  for (int u = 0; u < NSUB; ++u)
#pragma unroll
    for (int st = 0; st < CS; ++st)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        dv[t] = M::mma(Gc->tfrag(32 * t, st, lane, 32 * u), pf[u][st], dv[t]);
        dk[t] = M::mma(Qc->tfrag(32 * t, st, lane, 32 * u), sf[u][st], dk[t]);
      }
}

}  // namespace attn
