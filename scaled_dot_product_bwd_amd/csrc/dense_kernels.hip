// dense_kernels.hip -- the three gfx950 kernels of the dense attention backward.
//
//   k_row_stats  query-block-major, once per row: m, l = sum exp(s - m) and
//                delta = rowsum(P * dP), the latter as dY . O with O = P V
//                accumulated online (equal in exact arithmetic).  The
//                statistics triple is the one ruDNN ordered_kernel.rs
//                `history_backward` consumes (max, denominator, delta).
//   k_kv_bwd     KV-block-major: per 128-key block, over its visible query
//                chunks (64 rows bf16, 32 fp32) in ascending order,
//                recompute S and P, then
//                dV += P^T dY, dP = dY V^T, dS = P (dP - delta) scale,
//                dK += dS^T Q.  dK / dV stay in registers; one store at the end.
//   k_dq_bwd     query-block-major: per 128-query block, over its visible
//                32-key chunks in ascending order, S, P, dP, dS, dQ += dS K.
//                A dQ row has one owner, so no atomics are needed.
// The math is rlx-cpu 0.2.17 src/attention_bwd.rs `backward_dense_head_all`
// (one score / softmax recompute feeding all three gradients); the masks are
// its `apply_synthetic_mask` and Custom / Bias branches.
//
// Every workgroup has 4 waves; wave w owns 32 consecutive rows of the block.
// All five contractions run on 32x32 MFMA tiles (device_common.hpp).  The
// streamed operand (Q / dY chunks, or K / V chunks) is triple-buffered in LDS:
// while chunk c is consumed from one buffer, chunk c + 1 is landing in the
// second and chunk c + 2 is being requested into the third (bf16: direct
// global -> LDS loads), so each chunk costs one barrier and HBM / L2 latency
// stays hidden behind two chunks of compute.
#include "device_common.hpp"
#include "kv_core.hpp"
#include "launch.hpp"

namespace attn {

// Each kernel's chunk loop runs in a force-inlined `*_run` function unrolled by
// three, so every step has its LDS buffers fixed at compile time.  Steps are
// unconditional (a conditional step would make the accumulators merge across
// paths, which the compiler pays for with register copies); chunks no row of
// a wave sees are computed like any other and contribute P = 0.

// After the compute of a step: make this wave's loads of the next chunk land
// (leaving the `issued` loads of the chunk after it in flight), then hand the
// buffers over.  fp32 tiles are written from registers in complete() instead.
template <bool DIRECT, int PER_CHUNK>
__device__ __forceinline__ void end_step(bool issued) {
  if constexpr (DIRECT) {
    if (issued)
      wait_vmem_le<PER_CHUNK>();
    else
      wait_vmem();
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Row statistics.
template <typename T, int D> struct RowStatsState {
  typedef MT<T> M;
  static constexpr int NSD = D / M::KS, NT = D / 32;
  typename M::frag qf[NSD];
  f32x16 o[NT];
  float m_run, l_run;
  ChunkIO<T, D> io_k, io_v;
  const T *kbase, *vbase;
  int b, h, iw, qi, lane, l32, half, c_last;
};

template <typename T, int D, int MODE>
__device__ __forceinline__ void row_stats_step(const DenseParams &p, RowStatsState<T, D> &S, int c,
                                               const Tile<T, D> *Kc, const Tile<T, D> *Vc, int cn,
                                               Tile<T, D> *Kn, Tile<T, D> *Vn) {
  typedef MT<T> M;
  constexpr int NSD = D / M::KS, NT = D / 32, CS = M::CSTEPS;
  const int j0 = c * 32;
  const bool issued = cn <= S.c_last;
  if (issued) {
    S.io_k.issue(S.kbase, p.ks[1], cn * 32, p.Sk, *Kn);
    S.io_v.issue(S.vbase, p.vs[1], cn * 32, p.Sk, *Vn);
  }
  const bool check = MODE != MODE_INDEX || !tile_all_visible(p, S.iw, j0);
  // S^T = K Q^T: rows = keys (A from LDS), columns = this lane's query.
  typename M::frag ka[NSD];
#pragma unroll
  for (int s = 0; s < NSD; ++s) ka[s] = Kc->frag(S.l32, s, S.half);
  f32x16 sacc = f32x16{};
#pragma unroll
  for (int s = 0; s < NSD; ++s) sacc = M::mma(ka[s], S.qf[s], sacc);

  float sc[16];
  const int qi = S.qi, half = S.half;
  scores16<MODE>(p, sacc, sc, S.b, S.h, check, [&](int) { return qi; },
                 [&](int r) { return j0 + kr(r, half); });
  float mloc = sc[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, sc[r]);
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  const float m_new = fmaxf(S.m_run, mloc);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = fast_exp2(S.m_run - m_use);
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sc[r] = fast_exp2(sc[r] - m_use);
    psum += sc[r];
  }
  S.l_run = S.l_run * alpha + psum;
  S.m_run = m_new;
#pragma unroll
  for (int t = 0; t < NT; ++t) S.o[t] *= alpha;

  // O^T += V^T P^T: A = V read transposed from LDS, B = P straight from the S^T tile.
#pragma unroll
  for (int st = 0; st < CS; ++st) {
    const typename M::frag pf = creuse<T>(sc, st);
#pragma unroll
    for (int t = 0; t < NT; ++t) S.o[t] = M::mma(Vc->tfrag(32 * t, st, S.lane), pf, S.o[t]);
  }
  if (issued) {
    S.io_k.complete(*Kn);
    S.io_v.complete(*Vn);
  }
  end_step<ChunkIO<T, D>::DIRECT, 2 * ChunkIO<T, D>::LOADS>(issued);
}

template <typename T, int D, int MODE>
__device__ __forceinline__ void row_stats_run(const DenseParams &p, RowStatsState<T, D> &S,
                                              int c_first, Tile<T, D> *__restrict__ K0,
                                              Tile<T, D> *__restrict__ K1,
                                              Tile<T, D> *__restrict__ K2,
                                              Tile<T, D> *__restrict__ V0,
                                              Tile<T, D> *__restrict__ V1,
                                              Tile<T, D> *__restrict__ V2) {
  const int c_last = S.c_last;
  if (c_first <= c_last) {
    S.io_k.issue(S.kbase, p.ks[1], c_first * 32, p.Sk, *K0);
    S.io_v.issue(S.vbase, p.vs[1], c_first * 32, p.Sk, *V0);
    S.io_k.complete(*K0);
    S.io_v.complete(*V0);
  }
  const bool second = c_first + 1 <= c_last;
  if (second) {
    S.io_k.issue(S.kbase, p.ks[1], (c_first + 1) * 32, p.Sk, *K1);
    S.io_v.issue(S.vbase, p.vs[1], (c_first + 1) * 32, p.Sk, *V1);
    S.io_k.complete(*K1);
    S.io_v.complete(*V1);
  }
  end_step<ChunkIO<T, D>::DIRECT, 2 * ChunkIO<T, D>::LOADS>(second);
  int c = c_first;
  for (; c + 2 <= c_last; c += 3) {
    row_stats_step<T, D, MODE>(p, S, c, K0, V0, c + 2, K2, V2);
    row_stats_step<T, D, MODE>(p, S, c + 1, K1, V1, c + 3, K0, V0);
    row_stats_step<T, D, MODE>(p, S, c + 2, K2, V2, c + 4, K1, V1);
  }
  if (c <= c_last) row_stats_step<T, D, MODE>(p, S, c, K0, V0, c + 2, K2, V2);
  if (c + 1 <= c_last) row_stats_step<T, D, MODE>(p, S, c + 1, K1, V1, c + 3, K0, V0);
}

template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_row_stats(const DenseParams p) {
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NT = D / 32;
  __shared__ Tile<T, D> Ks0, Ks1, Ks2, Vs0, Vs1, Vs2;

  RowStatsState<T, D> S;
  const int tid = threadIdx.x, w = tid >> 6;
  S.lane = tid & 63;
  S.l32 = S.lane & 31;
  S.half = S.lane >> 5;
  const int nb = p.nblk;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = nb - 1 - (L % nb);  // the heaviest causal blocks first
  S.h = (L / nb) % p.H;
  S.b = L / (nb * p.H);
  const int i0 = blk * 128;
  S.iw = i0 + 32 * w;
  S.qi = S.iw + S.l32;
  const int b = S.b, h = S.h, qi = S.qi, half = S.half;
  const bool qvalid = qi < p.Sq;

  const T *qrow = (const T *)p.q + b * p.qs[0] + (int64_t)(qvalid ? qi : 0) * p.qs[1] + h * p.qs[2];
#pragma unroll
  for (int s = 0; s < NSD; ++s) S.qf[s] = load_frag<T>(qrow, s * KS + half * KL, qvalid);

  S.kbase = (const T *)p.k + b * p.ks[0] + h * p.ks[2];
  S.vbase = (const T *)p.v + b * p.vs[0] + h * p.vs[2];
  const int ilast = min(i0 + 128, p.Sq) - 1;
  const int jlo = max(0, i0 + p.lo_off);
  const int jhi = min(p.Sk - 1, (int)min((int64_t)ilast + p.hi_off, (int64_t)kBig));
  const int c_first = jlo >> 5;
  S.c_last = jhi >= jlo ? jhi >> 5 : c_first - 1;

  S.m_run = -INFINITY;
  S.l_run = 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) S.o[t] = f32x16{};
  S.io_k.init();
  S.io_v.init();
  // Let the fragment loads above land before the first chunk load is issued,
  // so the compiler knows they are complete inside the loop (otherwise it
  // would wait for them there, and with them for the chunk loads in flight).
  wait_vmem();
  row_stats_run<T, D, MODE>(p, S, c_first, &Ks0, &Ks1, &Ks2, &Vs0, &Vs1, &Vs2);

  // delta = dY . O / l  (O^T tile: lane holds its query, d = 32 t + kr(r, half)).
  const float l_tot = S.l_run + __shfl_xor(S.l_run, 32);
  const T *grow = (const T *)p.dy + b * p.dys[0] + (int64_t)(qvalid ? qi : 0) * p.dys[1] + h * p.dys[2];
  float dsum = 0.f;
  if (qvalid) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * t + 8 * g + 4 * half;
#pragma unroll
        for (int e = 0; e < 4; ++e) dsum += (float)grow[d0 + e] * S.o[t][4 * g + e];
      }
  }
  dsum += __shfl_xor(dsum, 32);
  if (qvalid && half == 0) {
    const int64_t row = ((int64_t)b * p.H + h) * p.Sq + qi;
    const bool empty = !(l_tot > 0.f);
    p.st_m[row] = empty ? -INFINITY : S.m_run * kLn2;
    p.st_l[row] = empty ? 0.f : l_tot;
    p.st_delta[row] = empty ? 0.f : dsum / l_tot;
    p.st_lse2[row] = empty ? INFINITY : S.m_run + __log2f(l_tot);
  }
}

// ---------------------------------------------------------------------------
// dK / dV, KV-block-major.  A step covers ROWS = 32 * NSUB queries as NSUB
// independent 32-row sub-tiles (kv_core.hpp).

// Statistics of the ROWS rows of chunk i0 into LDS, [lse2 x ROWS | delta x ROWS]
// per wave copy: direct-to-LDS dword loads, each wave writing its own copy so
// that every wave issues the same number of loads (STAT_LOADS).  Rows past Sq
// repeat the last row; the index mask gives them P = 0.
template <int ROWS>
__device__ __forceinline__ void issue_row_stats(const DenseParams &p, int64_t srow0, int i0,
                                                float *st, int wave, int lane) {
  float *dst = st + 2 * ROWS * wave;
  if constexpr (ROWS == 32) {
    const int row = min(i0 + (lane & 31), p.Sq - 1);
    dma_lds4(dst, (lane < 32 ? p.st_lse2 : p.st_delta) + srow0 + row);
  } else {
    const int row = min(i0 + lane, p.Sq - 1);
    dma_lds4(dst, p.st_lse2 + srow0 + row);
    dma_lds4(dst + 64, p.st_delta + srow0 + row);
  }
}
template <int ROWS> constexpr int stat_loads() { return ROWS == 32 ? 1 : 2; }

template <typename T, int D> struct KvState {
  typedef MT<T> M;
  static constexpr int NSD = D / M::KS, NT = D / 32, ROWS = KvShape<T>::ROWS;
  typename M::frag kf[NSD], vf[NSD];
  f32x16 dk[NT], dv[NT];
  ChunkIO<T, D, ROWS> io_q, io_g;
  const T *qbase, *gbase;
  int64_t srow0;
  int b, h, jw, kj, wave, lane, l32, half, c_last;
};

template <typename T, int D, int MODE>
__device__ __forceinline__ void kv_issue(const DenseParams &p, KvState<T, D> &S, int c,
                                         Tile<T, D, KvShape<T>::ROWS> *Q,
                                         Tile<T, D, KvShape<T>::ROWS> *G, float *st) {
  constexpr int ROWS = KvShape<T>::ROWS;
  S.io_q.issue(S.qbase, p.qs[1], c * ROWS, p.Sq, *Q);
  S.io_g.issue(S.gbase, p.dys[1], c * ROWS, p.Sq, *G);
  issue_row_stats<ROWS>(p, S.srow0, c * ROWS, st, S.wave, S.lane);
}

template <typename T, int D, int MODE>
__device__ __forceinline__ void kv_step(const DenseParams &p, KvState<T, D> &S, int c,
                                        const Tile<T, D, KvShape<T>::ROWS> *Qc,
                                        const Tile<T, D, KvShape<T>::ROWS> *Gc,
                                        const float *st_c, int cn,
                                        Tile<T, D, KvShape<T>::ROWS> *Qn,
                                        Tile<T, D, KvShape<T>::ROWS> *Gn, float *st_n) {
  constexpr int ROWS = KvShape<T>::ROWS;
  constexpr int PER_CHUNK = 2 * ChunkIO<T, D, ROWS>::LOADS + stat_loads<ROWS>();
  const int i0 = c * ROWS;
  const bool issued = cn <= S.c_last;
  if (issued) kv_issue<T, D, MODE>(p, S, cn, Qn, Gn, st_n);
  const int kj = S.kj, half = S.half, jw = S.jw, b = S.b, h = S.h;
  kv_chunk<T, D>(S.kf, S.vf, S.dk, S.dv, Qc, Gc, st_c, st_c + ROWS, p.scale, S.lane,
                 [&](int u, const f32x16 &acc, float *sc) {
                   const bool check = MODE != MODE_INDEX || !tile_all_visible(p, i0 + 32 * u, jw);
                   scores16<MODE>(p, acc, sc, b, h, check,
                                  [&](int r) { return i0 + 32 * u + kr(r, half); },
                                  [&](int) { return kj; });
                 });
  if (issued) {
    S.io_q.complete(*Qn);
    S.io_g.complete(*Gn);
  }
  end_step<ChunkIO<T, D, ROWS>::DIRECT, PER_CHUNK>(issued);
}

template <typename T, int D, int MODE>
__device__ __forceinline__ void kv_run(const DenseParams &p, KvState<T, D> &S, int c_first,
                                       Tile<T, D, KvShape<T>::ROWS> *__restrict__ Q0,
                                       Tile<T, D, KvShape<T>::ROWS> *__restrict__ Q1,
                                       Tile<T, D, KvShape<T>::ROWS> *__restrict__ Q2,
                                       Tile<T, D, KvShape<T>::ROWS> *__restrict__ G0,
                                       Tile<T, D, KvShape<T>::ROWS> *__restrict__ G1,
                                       Tile<T, D, KvShape<T>::ROWS> *__restrict__ G2,
                                       float *__restrict__ s0, float *__restrict__ s1,
                                       float *__restrict__ s2) {
  constexpr int ROWS = KvShape<T>::ROWS;
  constexpr int PER_CHUNK = 2 * ChunkIO<T, D, ROWS>::LOADS + stat_loads<ROWS>();
  const int c_last = S.c_last;
  if (c_first <= c_last) {
    kv_issue<T, D, MODE>(p, S, c_first, Q0, G0, s0);
    S.io_q.complete(*Q0);
    S.io_g.complete(*G0);
  }
  const bool second = c_first + 1 <= c_last;
  if (second) {
    kv_issue<T, D, MODE>(p, S, c_first + 1, Q1, G1, s1);
    S.io_q.complete(*Q1);
    S.io_g.complete(*G1);
  }
  end_step<ChunkIO<T, D, ROWS>::DIRECT, PER_CHUNK>(second);
  int c = c_first;
  for (; c + 2 <= c_last; c += 3) {
    kv_step<T, D, MODE>(p, S, c, Q0, G0, s0, c + 2, Q2, G2, s2);
    kv_step<T, D, MODE>(p, S, c + 1, Q1, G1, s1, c + 3, Q0, G0, s0);
    kv_step<T, D, MODE>(p, S, c + 2, Q2, G2, s2, c + 4, Q1, G1, s1);
  }
  if (c <= c_last) kv_step<T, D, MODE>(p, S, c, Q0, G0, s0, c + 2, Q2, G2, s2);
  if (c + 1 <= c_last) kv_step<T, D, MODE>(p, S, c + 1, Q1, G1, s1, c + 3, Q0, G0, s0);
}

template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) void k_kv_bwd(const DenseParams p) {
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NT = D / 32, ROWS = KvShape<T>::ROWS;
  __shared__ Tile<T, D, ROWS> Qs0, Qs1, Qs2, Gs0, Gs1, Gs2;
  __shared__ __attribute__((aligned(16))) float st0[8 * ROWS], st1[8 * ROWS], st2[8 * ROWS];

  KvState<T, D> S;
  const int w = threadIdx.x >> 6;
  S.wave = __builtin_amdgcn_readfirstlane(w);
  S.lane = threadIdx.x & 63;
  S.l32 = S.lane & 31;
  S.half = S.lane >> 5;
  const int nb = p.nblk;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = L % nb;  // key block 0 sees the most queries under a causal mask
  S.h = (L / nb) % p.H;
  S.b = L / (nb * p.H);
  const int j0b = blk * 128;
  S.jw = j0b + 32 * w;
  S.kj = S.jw + S.l32;
  const int b = S.b, h = S.h, kj = S.kj, half = S.half;
  const bool kvalid = kj < p.Sk;

  const T *krow = (const T *)p.k + b * p.ks[0] + (int64_t)(kvalid ? kj : 0) * p.ks[1] + h * p.ks[2];
  const T *vrow = (const T *)p.v + b * p.vs[0] + (int64_t)(kvalid ? kj : 0) * p.vs[1] + h * p.vs[2];
#pragma unroll
  for (int s = 0; s < NSD; ++s) {
    S.kf[s] = load_frag<T>(krow, s * KS + half * KL, kvalid);
    S.vf[s] = load_frag<T>(vrow, s * KS + half * KL, kvalid);
  }

  S.qbase = (const T *)p.q + b * p.qs[0] + h * p.qs[2];
  S.gbase = (const T *)p.dy + b * p.dys[0] + h * p.dys[2];
  S.srow0 = ((int64_t)b * p.H + h) * p.Sq;
  const int jlast = min(j0b + 128, p.Sk) - 1;
  const int ilo = max(0, (int)max((int64_t)j0b - p.hi_off, (int64_t)0));
  const int ihi = min(p.Sq - 1, (int)min((int64_t)jlast - p.lo_off, (int64_t)kBig));
  const int c_first = ilo / ROWS;
  S.c_last = ihi >= ilo ? ihi / ROWS : c_first - 1;

#pragma unroll
  for (int t = 0; t < NT; ++t) S.dk[t] = S.dv[t] = f32x16{};
  S.io_q.init();
  S.io_g.init();
  wait_vmem();  // fragment loads complete before the loop (see k_row_stats)
  kv_run<T, D, MODE>(p, S, c_first, &Qs0, &Qs1, &Qs2, &Gs0, &Gs1, &Gs2, st0, st1, st2);

  if (!kvalid) return;
  T *dkrow = (T *)p.dk + b * p.dks[0] + (int64_t)kj * p.dks[1] + h * p.dks[2];
  T *dvrow = (T *)p.dv + b * p.dvs[0] + (int64_t)kj * p.dvs[1] + h * p.dvs[2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * t + 8 * g + 4 * half;
      if (p.need_dk)
        store4<T>(dkrow + d0, S.dk[t][4 * g], S.dk[t][4 * g + 1], S.dk[t][4 * g + 2], S.dk[t][4 * g + 3]);
      if (p.need_dv)
        store4<T>(dvrow + d0, S.dv[t][4 * g], S.dv[t][4 * g + 1], S.dv[t][4 * g + 2], S.dv[t][4 * g + 3]);
    }
}

// ---------------------------------------------------------------------------
// dQ, query-block-major.
template <typename T, int D> struct DqState {
  typedef MT<T> M;
  static constexpr int NSD = D / M::KS, NT = D / 32;
  typename M::frag qf[NSD], gf[NSD];
  f32x16 dq[NT];
  ChunkIO<T, D> io_k, io_v;
  const T *kbase, *vbase;
  float lse, del;
  int b, h, iw, qi, lane, l32, half, c_last;
};

template <typename T, int D, int MODE>
__device__ __forceinline__ void dq_step(const DenseParams &p, DqState<T, D> &S, int c,
                                        const Tile<T, D> *Kc, const Tile<T, D> *Vc, int cn,
                                        Tile<T, D> *Kn, Tile<T, D> *Vn) {
  typedef MT<T> M;
  constexpr int NSD = D / M::KS, NT = D / 32, CS = M::CSTEPS;
  const int j0 = c * 32;
  const bool issued = cn <= S.c_last;
  if (issued) {
    S.io_k.issue(S.kbase, p.ks[1], cn * 32, p.Sk, *Kn);
    S.io_v.issue(S.vbase, p.vs[1], cn * 32, p.Sk, *Vn);
  }
  const bool check = MODE != MODE_INDEX || !tile_all_visible(p, S.iw, j0);
  // S^T = K Q^T and dP^T = V dY^T: rows = keys, columns = this lane's query.
  typename M::frag ka[NSD], va[NSD];
#pragma unroll
  for (int s = 0; s < NSD; ++s) {
    ka[s] = Kc->frag(S.l32, s, S.half);
    va[s] = Vc->frag(S.l32, s, S.half);
  }
  f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
  for (int s = 0; s < NSD; ++s) {
    sacc = M::mma(ka[s], S.qf[s], sacc);
    pacc = M::mma(va[s], S.gf[s], pacc);
  }
  float sc[16], dsv[16];
  const int qi = S.qi, half = S.half;
  scores16<MODE>(p, sacc, sc, S.b, S.h, check, [&](int) { return qi; },
                 [&](int r) { return j0 + kr(r, half); });
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float pr = fast_exp2(sc[r] - S.lse);
    dsv[r] = pr * (pacc[r] - S.del) * p.scale;
  }
  // dQ^T += K^T dS^T: A = K read transposed from LDS, B = dS straight from the tile.
#pragma unroll
  for (int st = 0; st < CS; ++st) {
    const typename M::frag sf = creuse<T>(dsv, st);
#pragma unroll
    for (int t = 0; t < NT; ++t) S.dq[t] = M::mma(Kc->tfrag(32 * t, st, S.lane), sf, S.dq[t]);
  }
  if (issued) {
    S.io_k.complete(*Kn);
    S.io_v.complete(*Vn);
  }
  end_step<ChunkIO<T, D>::DIRECT, 2 * ChunkIO<T, D>::LOADS>(issued);
}

template <typename T, int D, int MODE>
__device__ __forceinline__ void dq_run(const DenseParams &p, DqState<T, D> &S, int c_first,
                                       Tile<T, D> *__restrict__ K0, Tile<T, D> *__restrict__ K1,
                                       Tile<T, D> *__restrict__ K2, Tile<T, D> *__restrict__ V0,
                                       Tile<T, D> *__restrict__ V1, Tile<T, D> *__restrict__ V2) {
  const int c_last = S.c_last;
  if (c_first <= c_last) {
    S.io_k.issue(S.kbase, p.ks[1], c_first * 32, p.Sk, *K0);
    S.io_v.issue(S.vbase, p.vs[1], c_first * 32, p.Sk, *V0);
    S.io_k.complete(*K0);
    S.io_v.complete(*V0);
  }
  const bool second = c_first + 1 <= c_last;
  if (second) {
    S.io_k.issue(S.kbase, p.ks[1], (c_first + 1) * 32, p.Sk, *K1);
    S.io_v.issue(S.vbase, p.vs[1], (c_first + 1) * 32, p.Sk, *V1);
    S.io_k.complete(*K1);
    S.io_v.complete(*V1);
  }
  end_step<ChunkIO<T, D>::DIRECT, 2 * ChunkIO<T, D>::LOADS>(second);
  int c = c_first;
  for (; c + 2 <= c_last; c += 3) {
    dq_step<T, D, MODE>(p, S, c, K0, V0, c + 2, K2, V2);
    dq_step<T, D, MODE>(p, S, c + 1, K1, V1, c + 3, K0, V0);
    dq_step<T, D, MODE>(p, S, c + 2, K2, V2, c + 4, K1, V1);
  }
  if (c <= c_last) dq_step<T, D, MODE>(p, S, c, K0, V0, c + 2, K2, V2);
  if (c + 1 <= c_last) dq_step<T, D, MODE>(p, S, c + 1, K1, V1, c + 3, K0, V0);
}

template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_dq_bwd(const DenseParams p) {
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NT = D / 32;
  __shared__ Tile<T, D> Ks0, Ks1, Ks2, Vs0, Vs1, Vs2;

  DqState<T, D> S;
  const int tid = threadIdx.x, w = tid >> 6;
  S.lane = tid & 63;
  S.l32 = S.lane & 31;
  S.half = S.lane >> 5;
  const int nb = p.nblk;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int blk = nb - 1 - (L % nb);
  S.h = (L / nb) % p.H;
  S.b = L / (nb * p.H);
  const int i0 = blk * 128;
  S.iw = i0 + 32 * w;
  S.qi = S.iw + S.l32;
  const int b = S.b, h = S.h, qi = S.qi, half = S.half;
  const bool qvalid = qi < p.Sq;

  const T *qrow = (const T *)p.q + b * p.qs[0] + (int64_t)(qvalid ? qi : 0) * p.qs[1] + h * p.qs[2];
  const T *grow = (const T *)p.dy + b * p.dys[0] + (int64_t)(qvalid ? qi : 0) * p.dys[1] + h * p.dys[2];
#pragma unroll
  for (int s = 0; s < NSD; ++s) {
    S.qf[s] = load_frag<T>(qrow, s * KS + half * KL, qvalid);
    S.gf[s] = load_frag<T>(grow, s * KS + half * KL, qvalid);
  }
  const int64_t srow = ((int64_t)b * p.H + h) * p.Sq + (qvalid ? qi : 0);
  S.lse = qvalid ? p.st_lse2[srow] : INFINITY;
  S.del = qvalid ? p.st_delta[srow] : 0.f;

  S.kbase = (const T *)p.k + b * p.ks[0] + h * p.ks[2];
  S.vbase = (const T *)p.v + b * p.vs[0] + h * p.vs[2];
  const int ilast = min(i0 + 128, p.Sq) - 1;
  const int jlo = max(0, i0 + p.lo_off);
  const int jhi = min(p.Sk - 1, (int)min((int64_t)ilast + p.hi_off, (int64_t)kBig));
  const int c_first = jlo >> 5;
  S.c_last = jhi >= jlo ? jhi >> 5 : c_first - 1;

#pragma unroll
  for (int t = 0; t < NT; ++t) S.dq[t] = f32x16{};
  S.io_k.init();
  S.io_v.init();
  wait_vmem();  // fragment and statistics loads complete before the loop (see k_row_stats)
  dq_run<T, D, MODE>(p, S, c_first, &Ks0, &Ks1, &Ks2, &Vs0, &Vs1, &Vs2);

  if (!qvalid) return;
  T *dqrow = (T *)p.dq + b * p.dqs[0] + (int64_t)qi * p.dqs[1] + h * p.dqs[2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4<T>(dqrow + 32 * t + 8 * g + 4 * half, S.dq[t][4 * g], S.dq[t][4 * g + 1],
                S.dq[t][4 * g + 2], S.dq[t][4 * g + 3]);
}

// ---------------------------------------------------------------------------
// Launchers: one instantiation per (element type, head dim, mask mode).

template <typename T, int D, int MODE>
static hipError_t launch_t(int stage, const DenseParams &p, int nblocks, hipStream_t stream) {
  if (stage == STAGE_ROW_STATS)
    hipLaunchKernelGGL((k_row_stats<T, D, MODE>), dim3(nblocks), dim3(256), 0, stream, p);
  else if (stage == STAGE_KV)
    hipLaunchKernelGGL((k_kv_bwd<T, D, MODE>), dim3(nblocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((k_dq_bwd<T, D, MODE>), dim3(nblocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_d(int stage, int mode, const DenseParams &p, int nblocks, hipStream_t s) {
  switch (mode) {
    case MODE_KEYPAD: return launch_t<T, D, MODE_KEYPAD>(stage, p, nblocks, s);
    case MODE_BIAS: return launch_t<T, D, MODE_BIAS>(stage, p, nblocks, s);
    default: return launch_t<T, D, MODE_INDEX>(stage, p, nblocks, s);
  }
}

template <typename T>
static hipError_t launch_dt(int stage, int D, int mode, const DenseParams &p, int nblocks,
                            hipStream_t s) {
  switch (D) {
    case 32: return launch_d<T, 32>(stage, mode, p, nblocks, s);
    case 64: return launch_d<T, 64>(stage, mode, p, nblocks, s);
    default: return launch_d<T, 128>(stage, mode, p, nblocks, s);
  }
}

hipError_t launch_dense_stage(int stage, bool bf16_in, int D, int mode, const DenseParams &p,
                              int nblocks, hipStream_t stream) {
  if (nblocks <= 0) return hipSuccess;
  return bf16_in ? launch_dt<bf16>(stage, D, mode, p, nblocks, stream)
                 : launch_dt<float>(stage, D, mode, p, nblocks, stream);
}

}  // namespace attn
