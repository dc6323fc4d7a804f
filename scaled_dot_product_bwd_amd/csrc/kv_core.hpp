// kv_core.hpp -- the per-chunk body shared by the dense and the paged dK / dV
// kernels.
//
// A wave owns 32 keys, one per lane column (l32); their K and V rows sit in
// registers as MFMA B operands, their dK^T and dV^T accumulators as C tiles
// (column = key, rows = head-dim slice of 32).  One call consumes a chunk of
// 32 * NSUB query rows staged in LDS (Q, dY tiles and the row statistics) as
// NSUB independent 32-row sub-tiles, following rlx-cpu 0.2.17
// src/attention_bwd.rs `backward_dense_head_all`:
//   A  S = Q K^T, dP = dY V^T              rows = queries, A operand from LDS
//   B  P = exp2(S * scale * log2 e - lse2)  lse2 = m log2 e + log2 l, per row
//      dS' = P (dP - delta)                 (the factor `scale` of dS is applied
//                                            to dK once, by the caller; -lse2 and
//                                            -delta are the accumulators' start)
// K and V sit in registers as loaded: nothing is computed from them before
// their first MFMA, so their loads go straight into the operand registers and
// all of a tile's loads are in flight at once.  NEGV: the caller has negated V
// once its loads landed (dP starts at +delta, the chain forms delta - dP, and
// dS' and so dK^T come out negated, which the caller's store undoes as
// 0 - scale * x, keeping a zero +0) -- this
// saves the negation of delta in every chunk.  The matrix core's internal sum
// is not exactly sign-symmetric, so dK may differ from the plain form in the
// last bits (same arithmetic otherwise; dV is unchanged).
//   C  dV^T += dY^T P,  dK^T += Q^T dS'     A read transposed from LDS, B = C reuse
//
// Schedule.  With one wave per SIMD nothing hides latency but the wave's own
// instruction order, so the body is written as an explicit software pipeline
// and fenced with scheduling barriers that the compiler keeps:
//   * a step's LDS operands (one per MFMA, two MFMAs a step) are read two
//     steps ahead (a ring of three fragment registers per operand), so an
//     MFMA rarely waits for the LDS; a deeper ring costs registers (AGPR
//     copies) and measured slower;
//   * phase B of sub-tile 0 is spread over phase A of sub-tile 1, and phase B
//     of sub-tile 1 over phase C of sub-tile 0, so the softmax VALU work issues
//     while the matrix core runs.
// Masking is decided per chunk by the caller: the unmasked body has no
// per-element test at all; the masked one adds the caller's log2-domain term
// (0, a bias, or -inf) to every score, branch-free.
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

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// adj(u, r): log2-domain term added to the score of element r of sub-tile u
// (query row 32 u + kr(r, half) of the chunk, key = this lane's column); only
// called when MASKED.  nls / dst: the chunk's per-row statistics in LDS (row i
// at [i]): nls = -lse2 / scale_log2 and dst = delta.
//
// DK is the width of the score's contraction (Q and K rows, dK), DV that of the
// value side (dY and V rows, dV); DV <= DK.  They differ for a latent key: the
// score runs over [latent | position key] while the value is the latent alone,
// so the last (DK - DV) / KS score steps have no dP partner and the last
// (DK - DV) / 32 dK tiles no dV partner.
//
// MERGE (a latent that is both key and value): dS is scaled by ds_scale before
// it is packed, and P^T dY accumulates into the same tiles as dS^T Q, so dk
// holds the latent's whole gradient (tiles below DV / 32) and the position
// key's (the rest); dv is not used.  Phase C then issues all P^T dY products of
// a 32-row step before its dS^T Q products, so two MFMAs into one tile are
// never adjacent.
// dma(k), k < NDMA: the caller's k-th direct-to-LDS load for a later chunk,
// issued at step k (phase-A steps, then phase-C steps).  A wave stalls on a vector-memory issue while the
// CU's memory pipe is busy with the other waves' loads; spread one per step,
// the stalls fall under the running MFMAs instead of in front of them.
struct NoDma {
  __device__ __forceinline__ void operator()(int) const {}
};

// NSUB: 32-row sub-tiles per chunk (KvShape's by default; a wide latent key
// takes one, so that three chunk buffers still fit in LDS).
template <typename T, int DK, int DV, bool MASKED, bool MERGE, int NDMA = 0,
          typename Adj, typename Dma = NoDma, bool NEGV = false, int NSUB = KvShape<T>::NSUB>
__device__ __forceinline__ void kv_chunk(const typename MT<T>::frag *kf,
                                         const typename MT<T>::frag *vf, f32x16 *dk, f32x16 *dv,
                                         const Tile<T, DK, 32 * NSUB> *Qc,
                                         const Tile<T, DV, 32 * NSUB> *Gc,
                                         const float *nls, const float *dst, float scale_log2,
                                         int lane, Adj adj, float ds_scale = 1.f, Dma dma = Dma()) {
  typedef MT<T> M;
  typedef typename M::frag F;
  static_assert(DV <= DK && DV % 32 == 0 && DK % 32 == 0, "widths");
  constexpr int NSD = DK / M::KS, NSV = DV / M::KS, NT = DK / 32, NTV = DV / 32, CS = M::CSTEPS;
  constexpr int NA = NSUB * NSD;    // phase-A steps (S, and dP while s < NSV)
  constexpr int NC = NSUB * CS * NT;  // phase-C steps (dK, and dV while t < NTV)
  constexpr int RING = 3;
  static_assert(NDMA <= NA + NC, "one load per step");
  const int l32 = lane & 31, half = lane >> 5;

  f32x16 sacc[NSUB], pacc[NSUB];
  float pv[NSUB][16], dsv[NSUB][16];

  // The row statistics enter through the accumulators' initial values: S
  // starts at -lse2 / scale_log2 and dP at -delta, so after phase A
  // sacc * scale_log2 is the log2-domain exponent and pacc is dP - delta.
  // Elements 4g .. 4g + 3 of a lane are rows 8g + 4 half + 0..3: plain vector
  // loads into the accumulators, once per sub-tile and a few steps before its
  // first MFMA (no LDS read, hence no wait on the operand prefetch, inside
  // phase B).
  auto init_acc = [&](int u) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int rb = 32 * u + 8 * g + 4 * half;
      const f32x4 nl4 = *reinterpret_cast<const f32x4 *>(&nls[rb]);
      const f32x4 dl4 = *reinterpret_cast<const f32x4 *>(&dst[rb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sacc[u][4 * g + i] = nl4[i];
        pacc[u][4 * g + i] = NEGV ? dl4[i] : -dl4[i];
      }
    }
  };

  // Phase B for elements [r0, r1) of sub-tile u (needs sacc[u] / pacc[u] done).
  auto softmax = [&](int u, int r0, int r1) {
#pragma unroll
    for (int r = r0; r < r1; ++r) {
      float t;
      if constexpr (MASKED)
        t = fmaf(sacc[u][r], scale_log2, adj(u, r));
      else
        t = sacc[u][r] * scale_log2;
      const float pr = fast_exp2(t);
      pv[u][r] = pr;
      const float pd = pacc[u][r];  // dP - delta
      if constexpr (MERGE)
        dsv[u][r] = (pr * ds_scale) * pd;
      else
        dsv[u][r] = pr * pd;
    }
  };

  // Phase A: S and dP.  Step a = (u, s) reads Q / dY row fragments.
  F qa[RING], ga[RING];
  auto load_a = [&](int a) {
    const int u = a / NSD, s = a % NSD;
    qa[a % RING] = Qc->frag(32 * u + l32, s, half);
    if (s < NSV) ga[a % RING] = Gc->frag(32 * u + l32, s, half);
  };
  init_acc(0);
#pragma unroll
  for (int a = 0; a < RING - 1 && a < NA; ++a) load_a(a);
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int u = a / NSD, s = a % NSD;
    sched_fence();
    if (a + RING - 1 < NA) load_a(a + RING - 1);
    if (a < NDMA) dma(a);
    // the next sub-tile's statistics, two steps before its first MFMA
    if (u + 1 < NSUB && s == NSD - 2) init_acc(u + 1);
    sacc[u] = M::mma(qa[a % RING], kf[s], sacc[u]);
    if (s < NSV) pacc[u] = M::mma(ga[a % RING], vf[s], pacc[u]);
    // Sub-tile u - 1 is complete: spread its softmax over this sub-tile's steps.
    if (NSUB > 1 && u >= 1) {
      constexpr int PER = (16 + NSD - 1) / NSD;
      const int r0 = s * PER, r1 = r0 + PER < 16 ? r0 + PER : 16;
      if (r0 < 16) softmax(u - 1, r0, r1);
    }
  }
  sched_fence();
  if constexpr (NSUB == 1) softmax(0, 0, 16);

  if constexpr (MERGE) {
    // Phase C, merged: op i of a (u, st) group is P^T dY into tile i for
    // i < NTV, then dS^T [Q] into tile i - NTV; one transposed fragment each.
    constexpr int NOP = NTV + NT, NCM = NSUB * CS * NOP;
    F tf[RING], pf[NSUB][CS], sf[NSUB][CS];
    auto load_m = [&](int c) {
      const int u = c / (CS * NOP), st = (c / NOP) % CS, i = c % NOP;
      tf[c % RING] = i < NTV ? Gc->tfrag(32 * i, st, lane, 32 * u)
                             : Qc->tfrag(32 * (i - NTV), st, lane, 32 * u);
    };
    auto pack_m = [&](int c) {
      const int u = c / (CS * NOP), st = (c / NOP) % CS;
      pf[u][st] = creuse<T>(pv[u], st);
      sf[u][st] = creuse<T>(dsv[u], st);
    };
#pragma unroll
    for (int c = 0; c < RING - 1 && c < NCM; ++c) load_m(c);
    pack_m(0);
#pragma unroll
    for (int c = 0; c < NCM; ++c) {
      const int u = c / (CS * NOP), st = (c / NOP) % CS, i = c % NOP;
      sched_fence();
      if (c + RING - 1 < NCM) load_m(c + RING - 1);
      if (NSUB > 1 && u == 0) {
        constexpr int PER = (16 + CS * NOP - 1) / (CS * NOP);
        const int k = c % (CS * NOP);
        const int r0 = k * PER, r1 = r0 + PER < 16 ? r0 + PER : 16;
        if (r0 < 16) softmax(NSUB - 1, r0, r1);
      }
      if (c + 1 < NCM && (c + 1) % NOP == 0) pack_m(c + 1);
      if (i < NTV)
        dk[i] = M::mma(tf[c % RING], pf[u][st], dk[i]);
      else
        dk[i - NTV] = M::mma(tf[c % RING], sf[u][st], dk[i - NTV]);
    }
    sched_fence();
    return;
  }

  // Phase C: dV and dK.  Step c = (u, st, t) reads two transposed fragments;
  // the packed P / dS' operands of a (u, st) are built one step before their
  // first MFMA.
  F ta[RING], tb[RING], pf[NSUB][CS], sf[NSUB][CS];
  auto load_c = [&](int c) {
    const int u = c / (CS * NT), st = (c / NT) % CS, t = c % NT;
    if (t < NTV) ta[c % RING] = Gc->tfrag(32 * t, st, lane, 32 * u);
    tb[c % RING] = Qc->tfrag(32 * t, st, lane, 32 * u);
  };
  auto pack = [&](int c) {
    const int u = c / (CS * NT), st = (c / NT) % CS;
    pf[u][st] = creuse<T>(pv[u], st);
    sf[u][st] = creuse<T>(dsv[u], st);
  };
#pragma unroll
  for (int c = 0; c < RING - 1 && c < NC; ++c) load_c(c);
  pack(0);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int u = c / (CS * NT), st = (c / NT) % CS, t = c % NT;
    sched_fence();
    if (c + RING - 1 < NC) load_c(c + RING - 1);
    if (NA + c < NDMA) dma(NA + c);
    // The last sub-tile's softmax runs under the first sub-tile's phase C.
    if (NSUB > 1 && u == 0) {
      constexpr int PER = (16 + CS * NT - 1) / (CS * NT);
      const int i = c % (CS * NT);
      const int r0 = i * PER, r1 = r0 + PER < 16 ? r0 + PER : 16;
      if (r0 < 16) softmax(NSUB - 1, r0, r1);
    }
    if (c + 1 < NC && (c + 1) % NT == 0) pack(c + 1);
    if (t < NTV) dv[t] = M::mma(ta[c % RING], pf[u][st], dv[t]);
    dk[t] = M::mma(tb[c % RING], sf[u][st], dk[t]);
  }
  sched_fence();
}

}  // namespace attn
