// sd_core.hpp -- the chunk step of the fused query-major pass: row statistics
// and dQ together (bf16), shared by the dense kernel (k_stats_dq) and the paged
// one (k_paged_sdq), which differ only in where a chunk's K / V rows come from
// and in the mask.
//
// Per 64-key chunk, after S^T and dP^T (phase A) and the online statistics
// (RowStat, reference mref):
//   A^T += K^T (P~ * (dP - dh))^T,   B^T += K^T P~^T,   P~ = 2^(s - mref),
// both products reading the same transposed K fragment.  In exact arithmetic
//   dQ_i = scale sum_j P_ij (dP_ij - delta_i) K_j = scale (A_i - delta_i B_i) / l_i
// with delta_i = dl_i / l_i (rlx-cpu `backward_dense_head_all`: dS = P (dP -
// rowsum(P dP)) scale, dQ = dS K), so the statistics need no pass of their
// own: four contractions per visible pair instead of the statistics pass's
// two plus the dQ pass's three, and K / V stream through LDS once.  When a
// row's mref moves, its A and B are rescaled with l.
// Rounding: A - delta B cancels where one key dominates a row (dP ~ delta), and
// the bf16 rounding of P~ dP would then dominate dQ.  So A carries
// A' = sum P~ (dP - dh) K with dh the running estimate of delta (this chunk
// included): each chunk first moves A' to the new estimate (A' += (dh_old -
// dh) B, fp32), then adds P~ (dP - dh) K, the difference formed in fp32 before
// the bf16 rounding as in the dQ pass.  After the last chunk dh is delta (the
// caller moves A' to the delta it stores).  The statistics use the
// row-statistics kernel's arithmetic over 64 keys at a time (one reference
// update, one dh move and one barrier per 64 keys); they equal that kernel's
// (32 keys at a time) up to rounding.
#pragma once

#include "device_common.hpp"
#include "q_core.hpp"

namespace attn {

constexpr int kSdRing = 3;  // fragment ring of the fused pass (reads RING - 1 steps ahead)
constexpr int kSdKeys = 64;  // keys per chunk: two 32-key sub-tiles per statistics update

// A wave's state, as a struct with these members (each kernel adds its own):
//   typename MT<T>::frag qf[D / KS], gf[D / KS];  its 32 rows' Q and dY
//   f32x16 acc_a[D / 32], acc_b[D / 32];          A' and B
//   RowStat st;  float dh;                        statistics, delta's estimate
//   int lane, half;
template <int NT, typename St> __device__ __forceinline__ void sd_init(St &S) {
  S.st.init();
  S.dh = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) S.acc_a[t] = S.acc_b[t] = f32x16{};
}
// A' moved from dh to delta (the epilogue: A' = A - delta B).
template <int NT, typename St> __device__ __forceinline__ void sd_settle(St &S, float delta) {
  const float shift = S.dh - delta;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) S.acc_a[t][r] = fmaf(shift, S.acc_b[t][r], S.acc_a[t][r]);
}

// ---------------------------------------------------------------------------
// The chunk step.  Per 64-key chunk (two 32-key sub-tiles u) the arithmetic is
//   S^T and dP^T chains (Q / dY fragments in registers, K / V from LDS);
//   the statistics: the max and the reference update, the exponentials p~ and
//     their sum, sum p~ dP, l and dl, the new estimate dh of delta;
//   p~ and p~ (dP - dh) packed to bf16 for phase C;
//   phase C: per tile t, A' += (dh_old - dh) B just before its first product
//     (so each tile's shift overlaps the previous tile's MFMAs), then B and A'
//     accumulate over the chunk's four 16-key steps, one transposed K fragment
//     per pair of products.
// At one wave per SIMD only the wave's own instruction order overlaps VALU work
// with MFMAs, so the step is deferred: step c runs
//   chunk c's S chains, with chunk c - 1's middle (the rest of its sums, dh,
//     its packed p~ (dP - dh)) in their shadows;
//   chunk c - 1's phase C, with chunk c's statistics that need only S (the
//     max, the reference, the exponentials and their sum, the packed p~);
//   chunk c's dP chains, with its sum p~ dP over sub-tile 0.
// Every row sees the same operations in the same order as a step that runs
// chunk c alone.  The caller keeps chunk c's K tile until step c + 1 has run
// (four K buffers; V needs three) and finishes the last chunk with sd_finish.
// What a step hands to the next:
template <typename T> struct SdCarry {
  static constexpr int NU = kSdKeys / 32, CS = MT<T>::CSTEPS;
  float pr[NU][16];    // p~ of the chunk
  f32x16 pacc[NU];     // its dP^T
  typename MT<T>::frag pf[NU][CS];  // p~ packed for phase C
  float ls, ds, al;    // sum p~, sum p~ dP so far (sub-tile 0), the rescale
  bool moved;
};

// The middle of the pending chunk, part k of sd_nmid(): sum p~ dP over the
// sub-tiles after the first (three pieces), then the sums and dh, then one
// packed operand per (sub-tile, step).  `shift` receives dh_old - dh.
constexpr int kSdMidSum = 3;
template <typename T, int D, typename St>
__device__ __forceinline__ void sd_mid_part(St &S, SdCarry<T> &X, typename MT<T>::frag (&uf)[kSdKeys / 32][MT<T>::CSTEPS],
                                            float &shift, int k) {
  constexpr int NU = kSdKeys / 32, CS = MT<T>::CSTEPS, NR = (NU - 1) * 16;
  if (k < kSdMidSum) {
    const int r0 = k * NR / kSdMidSum, r1 = (k + 1) * NR / kSdMidSum;
#pragma unroll
    for (int r = r0; r < r1; ++r) X.ds = fmaf(X.pr[1 + r / 16][r % 16], X.pacc[1 + r / 16][r % 16], X.ds);
    pin(X.ds);
  } else if (k == kSdMidSum) {
    S.st.l = fmaf(S.st.l, X.al, X.ls);
    S.st.dl = fmaf(S.st.dl, X.al, X.ds);
    const float l_tot = halves_sum(S.st.l);
    const float dl_tot = halves_sum(S.st.dl);
    const float dh = l_tot > 0.f ? dl_tot * __builtin_amdgcn_rcpf(l_tot) : 0.f;
    shift = S.dh - dh;
    S.dh = dh;
  } else {
    const int q = k - kSdMidSum - 1, u = q / CS, st = q % CS;
    float pd[16 / CS];
#pragma unroll
    for (int e = 0; e < 16 / CS; ++e)
      pd[e] = X.pr[u][st * (16 / CS) + e] * (X.pacc[u][st * (16 / CS) + e] - S.dh);
    uf[u][st] = creuse<T>(pd, 0);
    pin(uf[u][st]);  // packed here, not next to its first product
  }
}
template <typename T> constexpr int sd_nmid() { return kSdMidSum + 1 + (kSdKeys / 32) * MT<T>::CSTEPS; }

// The pending chunk's rescale of A' and B (rare after the first visible chunk:
// a wave-uniform branch).  It runs at the start of the step, so that the S
// steps, the middle and phase C form one block: with the branch between them
// the compiler sinks the middle into phase C.
template <typename T, int D, typename St>
__device__ __forceinline__ void sd_rescale(St &S, const SdCarry<T> &X) {
  if (__any(X.moved)) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      S.acc_a[t] *= X.al;
      S.acc_b[t] *= X.al;
    }
  }
}

// Phase C of the pending chunk (its K tile Kp, its packed operands pf / uf):
// per tile the shift just before its first product; extra(k) after step k's
// two products (other work for the MFMAs' shadows).
template <typename T, int D, typename St, typename Extra>
__device__ __forceinline__ void sd_phase_c(St &S, const Tile<T, D, kSdKeys> *Kp,
                                           const typename MT<T>::frag (&pf)[kSdKeys / 32][MT<T>::CSTEPS],
                                           const typename MT<T>::frag (&uf)[kSdKeys / 32][MT<T>::CSTEPS],
                                           float shift, Extra extra) {
  typedef MT<T> M;
  typedef typename M::frag F;
  constexpr int NT = D / 32, CS = M::CSTEPS, NU = kSdKeys / 32, RING = kSdRing, NC = NU * CS * NT;
  F kt[RING];
  auto loadc = [&](int k) {
    const int t = k % NT, st = (k / NT) % CS, u = k / (NT * CS);
    kt[k % RING] = Kp->tfrag(32 * t, st, S.lane, 32 * u);
  };
#pragma unroll
  for (int k = 0; k < RING - 1 && k < NC; ++k) loadc(k);
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int t = k % NT, st = (k / NT) % CS, u = k / (NT * CS);
    sched_fence();
    if (k + RING - 1 < NC) loadc(k + RING - 1);
    if (k < NT) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S.acc_a[t][r] = fmaf(shift, S.acc_b[t][r], S.acc_a[t][r]);
    }
    S.acc_b[t] = M::mma(kt[k % RING], pf[u][st], S.acc_b[t]);
    S.acc_a[t] = M::mma(kt[k % RING], uf[u][st], S.acc_a[t]);
    extra(k);
  }
  sched_fence();
}
template <typename T, int D> constexpr int sd_ncsteps() { return (kSdKeys / 32) * MT<T>::CSTEPS * (D / 32); }

// Chunk c (tiles Kc / Vc in LDS); with PREV, chunk c - 1's middle and phase C
// (its K tile Kp, its carry X) run here too; X leaves with chunk c's carry.
// MASKED is fixed per loop by the caller (a branch inside the step would split
// it into blocks and let the compiler move work out of the MFMA shadows it was
// placed in); the unmasked step is for chunks whose every (row, key) pair is
// visible, with cl > 0.  cl = scale log2 e; adj_of(u, r): the mask term (log2
// domain: 0, -inf or a bias) of element r of sub-tile u (MASKED only);
// dma(k), k < 2 LOADS: the caller's k-th direct-to-LDS load of a later chunk,
// one per S step.  The step ends by waiting for every vector-memory operation
// but the 2 LOADS issued in it, then a barrier.
template <typename T, int D, bool MASKED, bool PREV, typename St, typename Adj, typename Dma>
__device__ __forceinline__ void sd_body_deferred(St &S, float cl, const Tile<T, D, kSdKeys> *Kc,
                                                 const Tile<T, D, kSdKeys> *Vc,
                                                 const Tile<T, D, kSdKeys> *Kp, SdCarry<T> &X,
                                                 Adj adj_of, Dma dma) {
  typedef MT<T> M;
  typedef typename M::frag F;
  constexpr int CS = M::CSTEPS, NSD = D / M::KS, RING = kSdRing;
  constexpr int KC = kSdKeys, NU = KC / 32, L = ChunkIO<T, D, KC>::LOADS;
  constexpr int NA = 2 * NU * NSD, NH = NA / 2, NM = sd_nmid<T>(), NC = sd_ncsteps<T, D>();
  static_assert(2 * L <= NH, "the loads go out in the S steps");
  constexpr bool plain = !MASKED;
  const int l32 = S.lane & 31, half = S.half;
  if constexpr (PREV) sd_rescale<T, D>(S, X);

  F fr[RING];
  auto load = [&](int i) {  // step i < NH: K of sub-tile i % NU, else V
    const int ii = i < NH ? i : i - NH;
    const int u = i < NH ? ii % NU : ii / NSD, s = i < NH ? ii / NU : ii % NSD;
    fr[i % RING] = i < NH ? Kc->frag(32 * u + l32, s, half) : Vc->frag(32 * u + l32, s, half);
  };
#pragma unroll
  for (int i = 0; i < RING - 1; ++i) load(i);
  f32x16 sacc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) sacc[u] = f32x16{};
  F uf[NU][CS];
  float shift = 0.f;
  // The S chains of both sub-tiles interleaved, the pending chunk's middle in
  // their steps.
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    sched_fence();
    load(i + RING - 1);
    if (i < 2 * L) dma(i);
    const int u = i % NU, s = i / NU;
    sacc[u] = M::mma(fr[i % RING], S.qf[s], sacc[u]);
    if constexpr (PREV) {
#pragma unroll
      for (int k = i * NM / NH; k < (i + 1) * NM / NH; ++k) sd_mid_part<T, D>(S, X, uf, shift, k);
    }
  }

  // Chunk c's statistics, part k of NPART: parts below NPRE need only S
  //   k < NU: sub-tile k's scores and running max;  k = NU: the reference;
  //   then the exponentials four at a time (their sum as they come);
  //   then each sub-tile's p~ packed for phase C;
  // the last three need sub-tile 0's dP: its sum p~ dP in three pieces.
  // Every sum runs in the order of the plain loop.
  float s2[NU][16], pr[NU][16], mx = 0.f, mu = 0.f, al = 1.f, ls = 0.f, ds = 0.f;
  bool moved = false;
  F pf[NU][CS];
  f32x16 pacc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) pacc[u] = f32x16{};
  constexpr int KX = NU + 1, KP = KX + 4 * NU, NPRE = KP + NU, NPART = NPRE + 3;
  auto stat_part = [&](int k) {
    if (k < NU) {
      const int u = k;
      if constexpr (plain) {
        if (u == 0) mx = sacc[0][0];
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[u][r]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s2[u][r] = fmaf(sacc[u][r], cl, adj_of(u, r));
        if (u == 0) mx = s2[0][0];
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s2[u][r]);
      }
    } else if (k == NU) {
      mx = halves_max(mx);
      if constexpr (plain) mx *= cl;
      al = row_stat_ref(S.st, mx, moved, mu);
    } else if (k < KP) {
      const int q = k - KX, u = q / 4, r0 = 4 * (q % 4);
#pragma unroll
      for (int r = r0; r < r0 + 4; ++r) {
        if constexpr (plain)
          pr[u][r] = fast_exp2(fmaf(sacc[u][r], cl, -mu));
        else
          pr[u][r] = fast_exp2(s2[u][r] - mu);
        ls += pr[u][r];
      }
      pin(ls);
    } else if (k < NPRE) {
      const int u = k - KP;
#pragma unroll
      for (int st = 0; st < CS; ++st) {
        pf[u][st] = creuse<T>(pr[u], st);
        pin(pf[u][st]);
      }
    } else {
      const int r0 = (k - NPRE) * 16 / 3, r1 = (k - NPRE + 1) * 16 / 3;
#pragma unroll
      for (int r = r0; r < r1; ++r) ds = fmaf(pr[0][r], pacc[0][r], ds);
      pin(ds);
    }
  };
  // With a pending chunk, the S-only parts go under its phase C; the first
  // chunk spreads all parts over its dP steps.
  constexpr int PRE = PREV ? NPRE : 0;
  if constexpr (PREV)
    sd_phase_c<T, D>(S, Kp, X.pf, uf, shift, [&](int k) {
#pragma unroll
      for (int j = k * NPRE / NC; j < (k + 1) * NPRE / NC; ++j) stat_part(j);
    });
  else
    sched_fence();

  // The dP chains one sub-tile after the other; the remaining parts in their
  // steps (the sum p~ dP pieces once sub-tile 0's chain is done).
  constexpr int NREST = NPART - PRE, FROM = PREV ? NSD : 0;
#pragma unroll
  for (int i = NH; i < NA; ++i) {
    sched_fence();
    if (i + RING - 1 < NA) load(i + RING - 1);
    const int ii = i - NH, u = ii / NSD, s = ii % NSD;
    pacc[u] = M::mma(fr[i % RING], S.gf[s], pacc[u]);
    if (ii >= FROM) {
#pragma unroll
      for (int k = (ii - FROM) * NREST / (NH - FROM); k < (ii - FROM + 1) * NREST / (NH - FROM); ++k)
        stat_part(PRE + k);
    }
  }
  sched_fence();
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    X.pacc[u] = pacc[u];
#pragma unroll
    for (int r = 0; r < 16; ++r) X.pr[u][r] = pr[u][r];
#pragma unroll
    for (int st = 0; st < CS; ++st) X.pf[u][st] = pf[u][st];
  }
  X.ls = ls;
  X.ds = ds;
  X.al = al;
  X.moved = moved;
  wait_vmem_le<2 * L>();  // the chunk requested a step ago has landed
  __syncthreads();
}

// After the last chunk's step: its middle and phase C.
template <typename T, int D, typename St>
__device__ __forceinline__ void sd_finish(St &S, const Tile<T, D, kSdKeys> *Kp, SdCarry<T> &X) {
  typename MT<T>::frag uf[kSdKeys / 32][MT<T>::CSTEPS];
  float shift = 0.f;
  sd_rescale<T, D>(S, X);
#pragma unroll
  for (int k = 0; k < sd_nmid<T>(); ++k) sd_mid_part<T, D>(S, X, uf, shift, k);
  sd_phase_c<T, D>(S, Kp, X.pf, uf, shift, [](int) {});
}

}  // namespace attn
