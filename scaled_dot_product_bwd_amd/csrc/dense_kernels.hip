// dense_kernels.hip -- the gfx950 kernels of the dense attention backward.
// bf16 runs k_stats_dq then k_kv_bwd; fp32 runs k_row_stats, k_kv_bwd,
// k_dq_bwd.
//
//   k_row_stats  query-block-major, once per row: m, l = sum exp(s - m) and
//                delta = rowsum(P * dP), accumulated online with dP = dY V^T.
//                The statistics triple is the one ruDNN ordered_kernel.rs
//                `history_backward` consumes (max, denominator, delta).
//   k_stats_dq   query-block-major (bf16): the row statistics and dQ in one
//                pass, dQ = scale (A - delta B) / l with A, B accumulated
//                against the running statistics (see its section).
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
// Every contraction runs on 32x32 MFMA tiles (device_common.hpp).  The
// streamed operand (Q / dY chunks, or K / V chunks) is triple-buffered in LDS:
// while chunk c is consumed from one buffer, chunk c + 1 is landing in the
// second and chunk c + 2 is being requested into the third (bf16: direct
// global -> LDS loads), so each chunk costs one barrier and HBM / L2 latency
// stays hidden behind two chunks of compute.
#include "device_common.hpp"
#include "kv_core.hpp"
#include "q_core.hpp"
#include "sd_core.hpp"
#include "launch.hpp"

namespace attn {

// Heads whose tiles an XCD interleaves (tile_order).  dQ: 4, which balances the
// causal block sizes as well as all of an XCD's heads and keeps the group's
// operands in L2.  dK / dV: all 8 of an XCD's heads, whose longest-first order
// balances best (149.7 us against 153.9 us with 2 and 152.9 us with 4, on the
// bf16 [4, 2048, 16, 128] causal workload) although it reads Q / dY about 1.5x
// from HBM.  The row statistics (three workgroups per CU) are fastest with all.
constexpr int kKvGroup = 8, kDqGroup = 4, kRsGroup = 8;

// The dQ kernel's chunk loop is unrolled by three, so every step has its LDS
// buffers fixed at compile time (no per-read address arithmetic); the row
// statistics, statistics + dQ and dK / dV rotate their buffers at run time
// (unrolled, the row statistics spill at three waves per SIMD; the others
// address their bodies with immediate offsets from one base anyway, and the
// fused pass keeps separate masked and unmasked loops).
// Steps are unconditional (a conditional step would make the accumulators merge
// across paths, which the compiler pays for with register copies); chunks no
// row of a wave sees are computed like any other and contribute P = 0.

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

// The query-major kernels' loads of a later K / V chunk cn, as a per-step hook
// for q_phase_a (direct loads only): load k < LOADS of K, then of V.  Past the
// last chunk the caller passes cn = c_last again (loaded into the free buffer,
// never read); the kernel drains the loads before it ends.
template <typename T, int D>
__device__ __forceinline__ auto q_next_chunk_dma(const DenseParams &p, ChunkIO<T, D> &io_k,
                                                 ChunkIO<T, D> &io_v, const T *kbase,
                                                 const T *vbase, int cn, Tile<T, D> &K,
                                                 Tile<T, D> &V) {
  constexpr int L = ChunkIO<T, D>::LOADS;
  const T *kc = kbase + (int64_t)cn * 32 * p.ks[1];
  const T *vc = vbase + (int64_t)cn * 32 * p.vs[1];
  const int last = p.Sk - 1 - cn * 32;
  const unsigned ksb = (unsigned)(p.ks[1] * sizeof(T)), vsb = (unsigned)(p.vs[1] * sizeof(T));
  return [=, &io_k, &io_v, &K, &V](int k) {
    if constexpr (ChunkIO<T, D>::DIRECT) {
      if (k < L)
        io_k.issue_one(k, kc, last, ksb, K);
      else
        io_v.issue_one(k - L, vc, last, vsb, V);
    }
  };
}

__device__ __forceinline__ void store_row_stat(const DenseParams &p, int64_t row, const RowStatOut &o) {
  p.st_m[row] = o.m;
  p.st_l[row] = o.l;
  p.st_delta[row] = o.delta;
  p.st_nls[row] = o.nls;
}

// The keys a query row sees by the index rule, [lo, lo + w]: key j is visible
// iff (unsigned)(j - lo) <= w, one compare per element (the same set as
// idx_visible).  A row past Sq, or one that sees no key, gets lo = INT_MAX,
// which no key index reaches (indices stay below 2^30 + 128, so j - lo does
// not overflow).  The bounds are formed in 64 bits: a padding row past Sq
// plus an offset of 2^30 would not fit in 32.
struct KeySpan {
  int lo;
  unsigned w;
};
__device__ __forceinline__ KeySpan key_span(const DenseParams &p, int qi) {
  const int64_t lo = max((int64_t)qi + p.lo_off, (int64_t)0);
  const int64_t hi = min((int64_t)qi + p.hi_off, (int64_t)p.Sk - 1);
  return (qi < p.Sq && hi >= lo) ? KeySpan{(int)lo, (unsigned)(hi - lo)} : KeySpan{INT_MAX, 0u};
}

// ---------------------------------------------------------------------------
// Row statistics.  Per query row: the denominator l = sum 2^(s - mref) and
// delta' = sum 2^(s - mref) dP against a lazily moved reference max (RowStat);
// at the end delta = delta' / l = rowsum(P * dP) (rlx-cpu
// `backward_dense_head_all`), with dP = dY V^T from phase A.
template <typename T, int D> struct RsState {
  typedef MT<T> M;
  static constexpr int NSD = D / M::KS, NQB = QShape<T>::NQB;
  typename M::frag qf[NQB][NSD], gf[NQB][NSD];
  RowStat st[NQB];
  int qi[NQB];
  KeySpan ks[NQB];  // the keys each row sees by the index rule
  ChunkIO<T, D> io_k, io_v;
  const T *kbase, *vbase;
  int b, h, lane, half, c_last, buf;
};

// Per-element mask term of (query qi, key kj), log2 domain (query-major
// kernels); ks = key_span(p, qi).
template <int MODE>
__device__ __forceinline__ float q_adj(const DenseParams &p, int b, int h, int qi, int kj,
                                       const KeySpan &ks) {
  if ((unsigned)(kj - ks.lo) > ks.w) return -INFINITY;
  if constexpr (MODE == MODE_INDEX) {
    return 0.f;
  } else {
    const float mv = p.mask[b * p.ms[0] + h * p.ms[1] + (int64_t)qi * p.ms[2] + (int64_t)kj * p.ms[3]];
    if constexpr (MODE == MODE_KEYPAD)
      return mv < p.thr ? -INFINITY : 0.f;
    else
      return mv * kLog2e;
  }
}

template <typename T, int D, int MODE, int NBUF>
__device__ __forceinline__ void rs_step(const DenseParams &p, RsState<T, D> &S, int c,
                                        Tile<T, D> *Ks, Tile<T, D> *Vs, bool masked) {
  constexpr int NQB = QShape<T>::NQB;
  const int bc = S.buf, bn = (bc + NBUF - 1) % NBUF;  // chunk c + NBUF - 1 goes to bn
  const bool issued = c + NBUF - 1 <= S.c_last;
  constexpr bool SPREAD = ChunkIO<T, D>::DIRECT;
  auto dma = q_next_chunk_dma<T, D>(p, S.io_k, S.io_v, S.kbase, S.vbase,
                                    min(c + NBUF - 1, S.c_last), Ks[bn], Vs[bn]);
  if (!SPREAD && issued) {
    S.io_k.issue(S.kbase, p.ks[1], (c + NBUF - 1) * 32, p.Sk, Ks[bn]);
    S.io_v.issue(S.vbase, p.vs[1], (c + NBUF - 1) * 32, p.Sk, Vs[bn]);
  }
  f32x16 sacc[NQB], pacc[NQB];
  q_phase_a<T, D, NQB, SPREAD ? 2 * ChunkIO<T, D>::LOADS : 0>(&Ks[bc], &Vs[bc], S.qf, S.gf, sacc,
                                                              pacc, S.lane, dma);
  const int j0 = c * 32, half = S.half;
  const bool plain = MODE == MODE_INDEX && !masked && p.scale_log2 > 0.f;
#pragma unroll
  for (int q = 0; q < NQB; ++q) {
    float pr[16];
    bool moved;
    row_stat_chunk(S.st[q], sacc[q], pacc[q], p.scale_log2, plain,
                   [&](int r) { return q_adj<MODE>(p, S.b, S.h, S.qi[q], j0 + kr(r, half), S.ks[q]); },
                   pr, moved);
  }
  if (issued) {
    S.io_k.complete(Ks[bn]);
    S.io_v.complete(Vs[bn]);
  }
  // With two buffers the chunk issued here is the next one: wait for all of it.
  end_step<ChunkIO<T, D>::DIRECT, 2 * ChunkIO<T, D>::LOADS>((SPREAD || issued) && NBUF == 3);
  S.buf = bc == NBUF - 1 ? 0 : bc + 1;
}

// Prologue shared by the query-major kernels: chunks c_first (and, with three
// buffers, c_first + 1) into buffers 0 (and 1).  It ends with a full drain, which
// also covers the register fragment loads issued before it: their latency and
// the first chunks' overlap, and the compiler knows them complete in the loop.
template <typename T, int D, int NBUF = 3>
__device__ __forceinline__ void q_prologue(const DenseParams &p, ChunkIO<T, D> &io_k,
                                           ChunkIO<T, D> &io_v, const T *kbase, const T *vbase,
                                           int c_first, int c_last, Tile<T, D> *Ks, Tile<T, D> *Vs) {
  if (c_first <= c_last) {
    io_k.issue(kbase, p.ks[1], c_first * 32, p.Sk, Ks[0]);
    io_v.issue(vbase, p.vs[1], c_first * 32, p.Sk, Vs[0]);
    io_k.complete(Ks[0]);
    io_v.complete(Vs[0]);
  }
  const bool second = NBUF == 3 && c_first + 1 <= c_last;
  if (second) {
    io_k.issue(kbase, p.ks[1], (c_first + 1) * 32, p.Sk, Ks[1]);
    io_v.issue(vbase, p.vs[1], (c_first + 1) * 32, p.Sk, Vs[1]);
    io_k.complete(Ks[1]);
    io_v.complete(Vs[1]);
  }
  wait_vmem();
  __syncthreads();
}

// Buffers of the row-statistics chunk stream.  Two (48 KB of LDS at D = 128)
// let three workgroups share a CU, three waves per SIMD, which hides more
// latency than a third buffer would.
constexpr int kRsBuf = 2;

// Key-axis piece of a split-form workgroup (piece 0 of the whole range
// otherwise): its chunks [lo, hi] inside the block's visible chunks [c0, c1].
struct QPiece {
  int piece, lo, hi;
};
template <bool SPLIT>
__device__ __forceinline__ QPiece q_piece(const DenseParams &p, int piece, int c0, int c1) {
  if constexpr (!SPLIT) return QPiece{0, c0, c1};
  return QPiece{piece, max(c0, piece * p.piece_chunks), min(c1, piece * p.piece_chunks + p.piece_chunks - 1)};
}

template <typename T, int D, int MODE, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_row_stats(const DenseParams p) {
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NQB = QShape<T>::NQB,
                QROWS = QShape<T>::QROWS;
  __shared__ Tile<T, D> Ks[kRsBuf], Vs[kRsBuf];

  RsState<T, D> S;
  const int tid = threadIdx.x, w = tid >> 6;
  S.lane = tid & 63;
  S.half = S.lane >> 5;
  const int l32 = S.lane & 31, half = S.half;
  const int nb = p.nblk;
  int bh, rank;
  // split form: consecutive workgroups are the pieces of one (block, head)
  const int np = SPLIT ? p.npiece : 1;
  tile_order<kRsGroup>(blockIdx.x / np, gridDim.x / np, nb, bh, rank);
  // the heaviest causal blocks first; under a narrow band the short first ones
  const int blk = narrow_band(p) ? rank : nb - 1 - rank;
  S.h = bh % p.H;
  S.b = bh / p.H;
  const int b = S.b, h = S.h;
  const int i0 = blk * QROWS;
#pragma unroll
  for (int q = 0; q < NQB; ++q) {
    const int qi = i0 + 32 * (NQB * w + q) + l32;
    S.qi[q] = qi;
    S.ks[q] = key_span(p, qi);
    const bool qvalid = qi < p.Sq;
    const T *qrow = (const T *)p.q + b * p.qs[0] + (int64_t)(qvalid ? qi : 0) * p.qs[1] + h * p.qs[2];
    const T *grow = (const T *)p.dy + b * p.dys[0] + (int64_t)(qvalid ? qi : 0) * p.dys[1] + h * p.dys[2];
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      S.qf[q][s] = load_frag<T>(qrow, s * KS + half * KL, qvalid);
      S.gf[q][s] = load_frag<T>(grow, s * KS + half * KL, qvalid);
    }
    S.st[q].init();
  }
  S.kbase = (const T *)p.k + b * p.ks[0] + (h / p.G) * p.ks[2];  // the head's K / V head
  S.vbase = (const T *)p.v + b * p.vs[0] + (h / p.G) * p.vs[2];
  const QRange R = q_range(p, i0, QROWS, MODE == MODE_INDEX);
  const QPiece Pc = q_piece<SPLIT>(p, (int)(blockIdx.x % np), R.c_first, R.c_last);
  S.c_last = Pc.hi;
  S.io_k.init(p.ks[1]);
  S.io_v.init(p.vs[1]);
  q_prologue<T, D, kRsBuf>(p, S.io_k, S.io_v, S.kbase, S.vbase, Pc.lo, Pc.hi, Ks, Vs);
  S.buf = 0;
  // Buffers rotate at run time here: unrolled by two (compile-time offsets)
  // the kernel spills at three waves per SIMD.
  for (int c = Pc.lo; c <= Pc.hi; ++c)
    rs_step<T, D, MODE, kRsBuf>(p, S, c, Ks, Vs, c < R.cu0 || c > R.cu1);
  wait_vmem();  // the repeated loads of the last step land before the workgroup ends

#pragma unroll
  for (int q = 0; q < NQB; ++q) {
    const int qi = S.qi[q];
    const int64_t row = ((int64_t)b * p.H + h) * p.Sq + qi;
    if constexpr (SPLIT) {
      // this piece's (mref, true max, l, delta') of the row, log2 domain
      const float l_tot = halves_sum(S.st[q].l);
      const float d_tot = halves_sum(S.st[q].dl);
      if (qi < p.Sq && half == 0)
        store4<float>(p.ws_split + 4 * ((int64_t)Pc.piece * p.B * p.H * p.Sq + row), S.st[q].mref,
                      S.st[q].mtrue, l_tot, d_tot);
    } else {
      const RowStatOut o = row_stat_final(S.st[q], p.inv_scale_log2);
      if (qi < p.Sq && half == 0) store_row_stat(p, row, o);
    }
  }
}

// The statistics of a row whose pieces were combined: M the common reference,
// mt the true max, l and dl (delta') relative to M; as row_stat_final forms
// them with M as the reference.
__device__ __forceinline__ RowStatOut merged_row_stat(float M, float mt, float l, float dl,
                                                      float inv_scale_log2) {
  RowStatOut o;
  o.empty = !(l > 0.f);
  o.m = o.empty ? -INFINITY : mt * kLn2;
  o.l = o.empty ? 0.f : l * fast_exp2(M - mt);
  o.delta = o.empty ? 0.f : dl / l;
  o.nls = (o.empty ? -INFINITY : -(M + __log2f(l))) * inv_scale_log2;
  o.inv_l = o.empty ? 0.f : 1.f / l;
  return o;
}

// Merge of the split row statistics: one thread per row, the pieces in order
// rescaled to their common reference M (the largest mref): l = sum 2^(mref_k
// - M) l_k and delta' likewise; then the statistics as row_stat_final forms
// them with M as the reference.
__global__ __launch_bounds__(256) void k_rs_merge(const DenseParams p) {
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  float M = -INFINITY, mt = -INFINITY;
  for (int k = 0; k < p.npiece; ++k) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(p.ws_split + 4 * (k * rows + row));
    M = fmaxf(M, v[0]);
    mt = fmaxf(mt, v[1]);
  }
  float l = 0.f, dl = 0.f;
  if (M != -INFINITY) {
    for (int k = 0; k < p.npiece; ++k) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(p.ws_split + 4 * (k * rows + row));
      const float a = fast_exp2(v[0] - M);  // 0 for a piece that saw nothing
      l = fmaf(v[2], a, l);
      dl = fmaf(v[3], a, dl);
    }
  }
  store_row_stat(p, row, merged_row_stat(M, mt, l, dl, p.inv_scale_log2));
}

// ---------------------------------------------------------------------------
// dK / dV, KV-block-major.  A step covers ROWS = 32 * NSUB queries as NSUB
// independent 32-row sub-tiles (kv_core.hpp).

// Statistics of the ROWS rows of chunk i0 into LDS, [-lse2 / scale_log2 x ROWS | delta x ROWS]
// per wave copy: direct-to-LDS dword loads, each wave writing its own copy so
// that every wave issues the same number of loads (STAT_LOADS).  Rows past Sq
// repeat the last row; the index mask gives them P = 0.
template <int ROWS>
__device__ __forceinline__ void issue_row_stats(const DenseParams &p, int64_t srow0, int i0,
                                                float *st, int wave, int lane) {
  float *dst = st + 2 * ROWS * wave;
  if constexpr (ROWS == 32) {
    const int row = min(i0 + (lane & 31), p.Sq - 1);
    dma_lds4(dst, (lane < 32 ? p.st_nls : p.st_delta) + srow0 + row);
  } else {
    const int row = min(i0 + lane, p.Sq - 1);
    dma_lds4(dst, p.st_nls + srow0 + row);
    dma_lds4(dst + 64, p.st_delta + srow0 + row);
  }
}
// The same into the copy at LDS byte address st_lds (of wave 0's copy).
template <int ROWS>
__device__ __forceinline__ void issue_row_stats_at(const DenseParams &p, int64_t srow0, int i0,
                                                   unsigned st_lds, int wave, int lane) {
  const unsigned dst = st_lds + 4u * 2 * ROWS * wave;
  if constexpr (ROWS == 32) {
    const int row = min(i0 + (lane & 31), p.Sq - 1);
    dma_lds4_at(dst, (lane < 32 ? p.st_nls : p.st_delta) + srow0 + row);
  } else {
    const int row = min(i0 + lane, p.Sq - 1);
    dma_lds4_at(dst, p.st_nls + srow0 + row);
    dma_lds4_at(dst + 4u * 64, p.st_delta + srow0 + row);
  }
}
template <int ROWS> constexpr int stat_loads() { return ROWS == 32 ? 1 : 2; }

template <typename T, int D> struct KvState {
  typedef MT<T> M;
  static constexpr int NSD = D / M::KS, NT = D / 32, ROWS = KvShape<T>::ROWS;
  typename M::frag kf[NSD], vf[NSD];
  f32x16 dk[NT], dv[NT];
  ChunkIO<T, D, ROWS> io_q, io_g;
  const T *qbase, *gbase;  // Q, dY of the group's first query head
  int64_t srow0;           // statistics row of (b, first query head, 0)
  int b, h0, jw, kj, wave, lane, l32, half, c_first, nch, total, buf;
  // Stream chunk min(v + 2, total - 1) while step v runs: its chunk index, its
  // Q / dY chunk start and its head's statistics row; advanced by one chunk per
  // step (dq_c, dg_c elements), or to the next head's first chunk (dq_w, dg_w).
  int nc;
  const T *qn, *gn;
  int64_t srn, dq_c, dq_w, dg_c, dg_w;
  KeySpan rows;  // the query rows that see key kj by the index rule (as a span)
};

// Chunks are numbered over the whole group: v = head * nch + (c - c_first) for
// the group's query heads in order, so the stream runs on across heads.
template <typename T, int D, int MODE>
__device__ __forceinline__ void kv_issue(const DenseParams &p, KvState<T, D> &S, int v,
                                         Tile<T, D, KvShape<T>::ROWS> *Q,
                                         Tile<T, D, KvShape<T>::ROWS> *G, float *st) {
  constexpr int ROWS = KvShape<T>::ROWS;
  const int hi = v / S.nch, c = S.c_first + (v - hi * S.nch);
  S.io_q.issue(S.qbase + hi * p.qs[2], p.qs[1], c * ROWS, p.Sq, *Q);
  S.io_g.issue(S.gbase + hi * p.dys[2], p.dys[1], c * ROWS, p.Sq, *G);
  issue_row_stats<ROWS>(p, S.srow0 + (int64_t)hi * p.Sq, c * ROWS, st, S.wave, S.lane);
}

// One chunk: request chunk c + 2, consume chunk c (MASKED: with the per-element
// mask term), hand over.  Buffers rotate at run time: chunk c sits in buffer
// S.buf, chunk c + 2 goes to the buffer chunk c - 1 used.
template <typename T, int D, int MODE, bool MASKED>
__device__ __forceinline__ void kv_step(const DenseParams &p, KvState<T, D> &S, int v, int c, int h,
                                        Tile<T, D, KvShape<T>::ROWS> *Qs,
                                        Tile<T, D, KvShape<T>::ROWS> *Gs, float (*st)[8 * KvShape<T>::ROWS]) {
  constexpr int ROWS = KvShape<T>::ROWS;
  constexpr int PER_CHUNK = 2 * ChunkIO<T, D, ROWS>::LOADS + stat_loads<ROWS>();
  const int bc = S.buf, bn = bc == 0 ? 2 : bc - 1;
  const int i0 = c * ROWS;
  const bool issued = v + 2 < S.total;
  // Chunk v + 2: with direct loads, one load per step of this chunk (the
  // kv_chunk dma hook), branch-free: past the end of the stream the last chunk
  // is loaded again into the free buffer (never read; drained by kv_run), so
  // every step issues the same loads.  With register loads (fp32) all of them
  // are issued here.
  constexpr bool SPREAD = ChunkIO<T, D, ROWS>::DIRECT;
  constexpr int LQ = ChunkIO<T, D, ROWS>::LOADS;
  const int cn = S.nc;  // stream chunk min(v + 2, total - 1)
  const int lastn = p.Sq - 1 - cn * ROWS;
  // LDS byte addresses of buffer bn as integers (bn is known only at run time)
  constexpr unsigned TB = sizeof(Tile<T, D, ROWS>), SB = sizeof(st[0]);
  const unsigned qlds = lds_addr(Qs) + bn * TB, glds = lds_addr(Gs) + bn * TB;
  const unsigned slds = lds_addr(st) + bn * SB;
  auto dma = [&](int k) {
    if constexpr (SPREAD) {
      if (k < LQ)
        S.io_q.issue_one_at(k, S.qn, lastn, (unsigned)(p.qs[1] * 2), qlds);
      else if (k < 2 * LQ)
        S.io_g.issue_one_at(k - LQ, S.gn, lastn, (unsigned)(p.dys[1] * 2), glds);
      else if (k == 2 * LQ)
        issue_row_stats_at<ROWS>(p, S.srn, cn * ROWS, slds, S.wave, S.lane);
    }
  };
  if (!SPREAD && issued) kv_issue<T, D, MODE>(p, S, v + 2, &Qs[bn], &Gs[bn], st[bn]);
  const int kj = S.kj, half = S.half, b = S.b;
  // Per-element mask term: the index rule, then padding or bias (log2 domain).
  auto adj = [&](int u, int r) -> float {
    const int i = i0 + 32 * u + kr(r, half);
    if ((unsigned)(i - S.rows.lo) > S.rows.w) return -INFINITY;
    if constexpr (MODE == MODE_INDEX) {
      return 0.f;
    } else {
      const float mv = p.mask[b * p.ms[0] + h * p.ms[1] + (int64_t)i * p.ms[2] + (int64_t)kj * p.ms[3]];
      if constexpr (MODE == MODE_KEYPAD)
        return mv < p.thr ? -INFINITY : 0.f;
      else
        return mv * kLog2e;
    }
  };
  const float *stc = st[bc];
  kv_chunk<T, D, D, MASKED, false, SPREAD ? 2 * LQ + 1 : 0, decltype(adj), decltype(dma), true>(
      S.kf, S.vf, S.dk, S.dv, &Qs[bc], &Gs[bc], stc, stc + ROWS, p.scale_log2, S.lane, adj, 1.f,
      dma);
  if (issued) {
    S.io_q.complete(Qs[bn]);
    S.io_g.complete(Gs[bn]);
  }
  end_step<ChunkIO<T, D, ROWS>::DIRECT, PER_CHUNK>(SPREAD || issued);
  S.buf = bc == 2 ? 0 : bc + 1;
  // Step v + 1 loads stream chunk min(v + 3, total - 1): the next chunk of the
  // head, or the next head's first.
  const bool adv = v + 3 < S.total, wrap = S.nc == S.c_first + S.nch - 1;
  if (adv) {  // wave-uniform
    S.nc = wrap ? S.c_first : S.nc + 1;
    S.qn += wrap ? S.dq_w : S.dq_c;
    S.gn += wrap ? S.dg_w : S.dg_c;
    S.srn += wrap ? (int64_t)p.Sq : 0;
  }
}

// All visible chunks of the block, in ascending order, for each query head of
// the group in turn.  Chunks every (query, key) pair of which the index rule
// keeps (the causal or window band's interior) run the unmasked body; the
// band's edges and padding / bias masks the masked one.  Each variant has its
// own loop, so no loop body holds both.
template <typename T, int D, int MODE>
__device__ __forceinline__ void kv_run(const DenseParams &p, KvState<T, D> &S, int c_last,
                                       int j0b, Tile<T, D, KvShape<T>::ROWS> *Qs,
                                       Tile<T, D, KvShape<T>::ROWS> *Gs,
                                       float (*st)[8 * KvShape<T>::ROWS]) {
  constexpr int ROWS = KvShape<T>::ROWS;
  const int c_first = S.c_first;
  if (S.total <= 0) return;
  kv_issue<T, D, MODE>(p, S, 0, &Qs[0], &Gs[0], st[0]);
  S.io_q.complete(Qs[0]);
  S.io_g.complete(Gs[0]);
  const bool second = S.total > 1;
  if (second) {
    kv_issue<T, D, MODE>(p, S, 1, &Qs[1], &Gs[1], st[1]);
    S.io_q.complete(Qs[1]);
    S.io_g.complete(Gs[1]);
  }
  // A full drain: also the K / V fragment loads issued before (their latency
  // overlaps the first chunks'; the compiler then knows them complete).  V is
  // negated now, once per tile, with every load landed (the body's NEGV form).
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int s = 0; s < KvState<T, D>::NSD; ++s) S.vf[s] = neg_frag<T>(S.vf[s]);
  S.buf = 0;
  {
    const int vn = min(2, S.total - 1), hn = vn / S.nch;
    S.nc = c_first + (vn - hn * S.nch);
    S.dq_c = (int64_t)ROWS * p.qs[1];
    S.dg_c = (int64_t)ROWS * p.dys[1];
    S.dq_w = p.qs[2] - (int64_t)(S.nch - 1) * S.dq_c;
    S.dg_w = p.dys[2] - (int64_t)(S.nch - 1) * S.dg_c;
    S.qn = S.qbase + hn * p.qs[2] + S.nc * S.dq_c;
    S.gn = S.gbase + hn * p.dys[2] + S.nc * S.dg_c;
    S.srn = S.srow0 + (int64_t)hn * p.Sq;
  }
  // Unmasked chunks [cu0, cu1]: every row i of the chunk sees every key j of the
  // block: j_last - i <= hi_off, j0 - i >= lo_off, i < Sq, j_last < Sk.
  int cu0 = c_last + 1, cu1 = c_last;
  if (MODE == MODE_INDEX && j0b + 128 <= p.Sk) {
    const int64_t lo_i = max((int64_t)j0b + 127 - p.hi_off, (int64_t)0);
    const int64_t hi_i = min((int64_t)j0b - p.lo_off, (int64_t)p.Sq - 1);
    cu0 = (int)min((lo_i + ROWS - 1) / ROWS, (int64_t)c_last + 1);
    cu1 = (int)min((hi_i + 1) / ROWS - 1, (int64_t)c_last);
    if (cu0 < c_first) cu0 = c_first;
    if (cu1 < cu0 - 1) cu1 = cu0 - 1;
  }
  for (int hi = 0; hi < p.G; ++hi) {
    const int h = S.h0 + hi, v0 = hi * S.nch - c_first;
    int c = c_first;
    for (; c < cu0; ++c) kv_step<T, D, MODE, true>(p, S, v0 + c, c, h, Qs, Gs, st);
    for (; c <= cu1; ++c) kv_step<T, D, MODE, false>(p, S, v0 + c, c, h, Qs, Gs, st);
    for (; c <= c_last; ++c) kv_step<T, D, MODE, true>(p, S, v0 + c, c, h, Qs, Gs, st);
  }
  wait_vmem();  // the repeated loads of the last steps land before the workgroup ends
}

template <typename T, int D, int MODE, bool SPLIT>
__global__ __launch_bounds__(256) void k_kv_bwd(const DenseParams p) {
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NT = D / 32, ROWS = KvShape<T>::ROWS;
  __shared__ Tile<T, D, ROWS> Qs[3], Gs[3];
  __shared__ __attribute__((aligned(16))) float st[3][8 * ROWS];

  KvState<T, D> S;
  const int w = threadIdx.x >> 6;
  S.wave = __builtin_amdgcn_readfirstlane(w);
  S.lane = threadIdx.x & 63;
  S.l32 = S.lane & 31;
  S.half = S.lane >> 5;
  const int nb = p.nblk;
  int bg, blk;  // key block 0 sees the most queries under a causal mask: rank = block
  // split form: consecutive workgroups are the query pieces of one key block
  const int np = SPLIT ? p.npiece : 1;
  tile_order<kKvGroup>(blockIdx.x / np, gridDim.x / np, nb, bg, blk);
  if (narrow_band(p)) blk = nb - 1 - blk;  // the short last key blocks first
  const int g = bg % p.Hkv;  // the K / V head; its query heads are g * G ... g * G + G - 1
  S.b = bg / p.Hkv;
  S.h0 = g * p.G;
  const int j0b = blk * 128;
  S.jw = j0b + 32 * w;
  S.kj = S.jw + S.l32;
  {  // rows i with lo_off <= kj - i <= hi_off, i < Sq, for kj < Sk (64-bit bounds)
    const int64_t lo = max((int64_t)S.kj - p.hi_off, (int64_t)0);
    const int64_t hi = min((int64_t)S.kj - p.lo_off, (int64_t)p.Sq - 1);
    S.rows = (S.kj < p.Sk && hi >= lo) ? KeySpan{(int)lo, (unsigned)(hi - lo)}
                                       : KeySpan{INT_MAX, 0u};
  }
  const int b = S.b, kj = S.kj, half = S.half;
  const bool kvalid = kj < p.Sk;

  const T *krow = (const T *)p.k + b * p.ks[0] + (int64_t)(kvalid ? kj : 0) * p.ks[1] + g * p.ks[2];
  const T *vrow = (const T *)p.v + b * p.vs[0] + (int64_t)(kvalid ? kj : 0) * p.vs[1] + g * p.vs[2];
#pragma unroll
  for (int s = 0; s < NSD; ++s) {
    S.kf[s] = load_frag<T>(krow, s * KS + half * KL, kvalid);
    S.vf[s] = load_frag<T>(vrow, s * KS + half * KL, kvalid);
  }

  S.qbase = (const T *)p.q + b * p.qs[0] + S.h0 * p.qs[2];
  S.gbase = (const T *)p.dy + b * p.dys[0] + S.h0 * p.dys[2];
  S.srow0 = ((int64_t)b * p.H + S.h0) * p.Sq;
  const int jlast = min(j0b + 128, p.Sk) - 1;
  const int ilo = max(0, (int)max((int64_t)j0b - p.hi_off, (int64_t)0));
  const int ihi = min(p.Sq - 1, (int)min((int64_t)jlast - p.lo_off, (int64_t)kBig));
  S.c_first = ilo / ROWS;
  int c_last = ihi >= ilo ? ihi / ROWS : S.c_first - 1;
  const QPiece Pc = q_piece<SPLIT>(p, (int)(blockIdx.x % np), S.c_first, c_last);
  S.c_first = Pc.lo;
  c_last = Pc.hi;
  S.nch = c_last - S.c_first + 1;
  S.total = S.nch > 0 ? S.nch * p.G : 0;

#pragma unroll
  for (int t = 0; t < NT; ++t) S.dk[t] = S.dv[t] = f32x16{};
  S.io_q.init(p.qs[1]);
  S.io_g.init(p.dys[1]);
  kv_run<T, D, MODE>(p, S, c_last, j0b, Qs, Gs, st);

  if constexpr (SPLIT) {
    // this piece's raw accumulators of the wave's keys (dK negated and without
    // its factor, dV), merged by k_kv_merge; 2 D floats per key row
    if (!kvalid) return;
    float *wrow = p.ws_split + ((int64_t)Pc.piece * p.B * p.Hkv * p.Sk +
                                ((int64_t)b * p.Hkv + g) * p.Sk + kj) * (2 * D);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d0 = 32 * t + 8 * q + 4 * half;
        store4<float>(wrow + d0, S.dk[t][4 * q], S.dk[t][4 * q + 1], S.dk[t][4 * q + 2],
                      S.dk[t][4 * q + 3]);
        store4<float>(wrow + D + d0, S.dv[t][4 * q], S.dv[t][4 * q + 1], S.dv[t][4 * q + 2],
                      S.dv[t][4 * q + 3]);
      }
    return;
  }

  // dK (times the factor of dS, applied once) and dV of the wave's 32 keys.
  typedef RowStore<T, D> RS;
  if constexpr (4 * RS::BYTES <= sizeof(Qs) && 4 * RS::BYTES <= sizeof(Gs)) {
    // whole rows through LDS (the chunk tiles are free once every wave is done)
    __syncthreads();
    char *lk = reinterpret_cast<char *>(Qs) + w * RS::BYTES;
    char *lv = reinterpret_cast<char *>(Gs) + w * RS::BYTES;
    if (p.need_dk) RS::template write_tiles<true>(S.dk, p.scale, lk, S.lane);  // dK was accumulated negated
    if (p.need_dv) RS::write_tiles(S.dv, 1.f, lv, S.lane);
    const int nvalid = max(0, min(32, p.Sk - S.jw));
    T *dk0 = (T *)p.dk + b * p.dks[0] + (int64_t)S.jw * p.dks[1] + g * p.dks[2];
    T *dv0 = (T *)p.dv + b * p.dvs[0] + (int64_t)S.jw * p.dvs[1] + g * p.dvs[2];
    if (p.need_dk) RS::store_rows(lk, nvalid, [&](int n) { return dk0 + (int64_t)n * p.dks[1]; }, S.lane);
    if (p.need_dv) RS::store_rows(lv, nvalid, [&](int n) { return dv0 + (int64_t)n * p.dvs[1]; }, S.lane);
  } else {
    if (!kvalid) return;
    T *dkrow = (T *)p.dk + b * p.dks[0] + (int64_t)kj * p.dks[1] + g * p.dks[2];
    T *dvrow = (T *)p.dv + b * p.dvs[0] + (int64_t)kj * p.dvs[1] + g * p.dvs[2];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * t + 8 * g + 4 * half;
        const float sc = p.scale;  // dK was accumulated negated: 0 - sc * x (a zero stays +0)
        if (p.need_dk)
          store4<T>(dkrow + d0, 0.f - sc * S.dk[t][4 * g], 0.f - sc * S.dk[t][4 * g + 1],
                    0.f - sc * S.dk[t][4 * g + 2], 0.f - sc * S.dk[t][4 * g + 3]);
        if (p.need_dv)
          store4<T>(dvrow + d0, S.dv[t][4 * g], S.dv[t][4 * g + 1], S.dv[t][4 * g + 2],
                    S.dv[t][4 * g + 3]);
      }
  }
}

// ---------------------------------------------------------------------------
// dQ, query-block-major: per chunk P = 2^(s - lse2), dS' = P (dP - delta) and
// dQ^T += K^T dS'^T (A = K read transposed from LDS, once per fragment for all
// query blocks); the factor `scale` of dS is applied at the store.
template <typename T, int D> struct DqState {
  typedef MT<T> M;
  static constexpr int NSD = D / M::KS, NT = D / 32, NQB = QShape<T>::NQB;
  typename M::frag qf[NQB][NSD], gf[NQB][NSD];
  f32x16 dq[NQB][NT];
  float nlse[NQB], del[NQB];
  int qi[NQB];
  KeySpan ks[NQB];  // the keys each row sees by the index rule
  ChunkIO<T, D> io_k, io_v;
  const T *kbase, *vbase;
  int b, h, lane, half, c_last, buf;
};

template <typename T, int D, int MODE, int BC>
__device__ __forceinline__ void dq_step(const DenseParams &p, DqState<T, D> &S, int c,
                                        Tile<T, D> *Ks, Tile<T, D> *Vs, bool masked) {
  typedef MT<T> M;
  constexpr int NT = D / 32, CS = M::CSTEPS, NQB = QShape<T>::NQB;
  constexpr int bc = BC, bn = (BC + 2) % 3;
  const bool issued = c + 2 <= S.c_last;
  constexpr bool SPREAD = ChunkIO<T, D>::DIRECT;
  auto dma = q_next_chunk_dma<T, D>(p, S.io_k, S.io_v, S.kbase, S.vbase, min(c + 2, S.c_last),
                                    Ks[bn], Vs[bn]);
  if (!SPREAD && issued) {
    S.io_k.issue(S.kbase, p.ks[1], (c + 2) * 32, p.Sk, Ks[bn]);
    S.io_v.issue(S.vbase, p.vs[1], (c + 2) * 32, p.Sk, Vs[bn]);
  }
  f32x16 sacc[NQB], pacc[NQB];
  q_phase_a<T, D, NQB, SPREAD ? 2 * ChunkIO<T, D>::LOADS : 0>(&Ks[bc], &Vs[bc], S.qf, S.gf, sacc,
                                                              pacc, S.lane, dma);
  const int j0 = c * 32, half = S.half;
  float dsv[NQB][16];
#pragma unroll
  for (int q = 0; q < NQB; ++q) {
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = fmaf(sacc[q][r], p.scale_log2, S.nlse[q]);
    if (MODE != MODE_INDEX || masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] += q_adj<MODE>(p, S.b, S.h, S.qi[q], j0 + kr(r, half), S.ks[q]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) dsv[q][r] = fast_exp2(t[r]) * (pacc[q][r] - S.del[q]);
  }
  const Tile<T, D> *Kc = &Ks[bc];
#pragma unroll
  for (int st = 0; st < CS; ++st) {
    typename M::frag sf[NQB];
#pragma unroll
    for (int q = 0; q < NQB; ++q) sf[q] = creuse<T>(dsv[q], st);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const typename M::frag kt = Kc->tfrag(32 * t, st, S.lane);
#pragma unroll
      for (int q = 0; q < NQB; ++q) S.dq[q][t] = M::mma(kt, sf[q], S.dq[q][t]);
    }
  }
  if (issued) {
    S.io_k.complete(Ks[bn]);
    S.io_v.complete(Vs[bn]);
  }
  end_step<ChunkIO<T, D>::DIRECT, 2 * ChunkIO<T, D>::LOADS>(SPREAD || issued);
}

template <typename T, int D, int MODE, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_dq_bwd(const DenseParams p) {
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NT = D / 32, NQB = QShape<T>::NQB,
                QROWS = QShape<T>::QROWS;
  __shared__ Tile<T, D> Ks[3], Vs[3];

  DqState<T, D> S;
  const int tid = threadIdx.x, w = tid >> 6;
  S.lane = tid & 63;
  S.half = S.lane >> 5;
  const int l32 = S.lane & 31, half = S.half;
  const int nb = p.nblk;
  int bh, rank;
  // split form (never with a forward's statistics): consecutive workgroups are
  // the pieces of one (block, head)
  const int np = SPLIT ? p.npiece : 1;
  tile_order<kDqGroup>(blockIdx.x / np, gridDim.x / np, nb, bh, rank);
  const int blk = narrow_band(p) ? rank : nb - 1 - rank;  // as in the statistics kernel
  S.h = bh % p.H;
  S.b = bh / p.H;
  const int b = S.b, h = S.h;
  const int i0 = blk * QROWS;
#pragma unroll
  for (int q = 0; q < NQB; ++q) {
    const int qi = i0 + 32 * (NQB * w + q) + l32;
    S.qi[q] = qi;
    S.ks[q] = key_span(p, qi);
    const bool qvalid = qi < p.Sq;
    const T *qrow = (const T *)p.q + b * p.qs[0] + (int64_t)(qvalid ? qi : 0) * p.qs[1] + h * p.qs[2];
    const T *grow = (const T *)p.dy + b * p.dys[0] + (int64_t)(qvalid ? qi : 0) * p.dys[1] + h * p.dys[2];
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      S.qf[q][s] = load_frag<T>(qrow, s * KS + half * KL, qvalid);
      S.gf[q][s] = load_frag<T>(grow, s * KS + half * KL, qvalid);
    }
    const int64_t srow = ((int64_t)b * p.H + h) * p.Sq + (qvalid ? qi : 0);
    if (p.fo != nullptr) {
      // From a forward's saved statistics: delta = dY . O (equal to rowsum(P *
      // dP) as O = P V), -lse2 = -L log2 e; both halves of the wave hold half
      // of the row's columns.  Published for the dK / dV pass, which follows.
      const T *orow = (const T *)p.fo + b * p.fos[0] + (int64_t)(qvalid ? qi : 0) * p.fos[1] +
                      h * p.fos[2];
      float dsum = 0.f;
#pragma unroll
      for (int s = 0; s < NSD; ++s) {
        const typename M::frag of = load_frag<T>(orow, s * KS + half * KL, qvalid);
        dsum += frag_dot<T>(S.gf[q][s], of);
      }
      dsum = halves_sum(dsum);
      const float L = qvalid ? p.flse[srow] : -INFINITY;
      const bool empty = !(L > -INFINITY);  // a row that sees no key: P = 0, delta = 0
      const float nls = (empty ? -INFINITY : -L * kLog2e) * p.inv_scale_log2;
      S.nlse[q] = nls * p.scale_log2;
      S.del[q] = empty ? 0.f : dsum;
      if (qvalid && half == 0) {
        p.st_delta[srow] = S.del[q];
        p.st_nls[srow] = nls;
      }
    } else {
      S.nlse[q] = qvalid ? p.st_nls[srow] * p.scale_log2 : -INFINITY;  // -lse2
      S.del[q] = qvalid ? p.st_delta[srow] : 0.f;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) S.dq[q][t] = f32x16{};
  }
  if (p.dq == nullptr) return;  // statistics only (a forward's, published above)

  S.kbase = (const T *)p.k + b * p.ks[0] + (h / p.G) * p.ks[2];  // the head's K / V head
  S.vbase = (const T *)p.v + b * p.vs[0] + (h / p.G) * p.vs[2];
  const QRange R = q_range(p, i0, QROWS, MODE == MODE_INDEX);
  const QPiece Pc = q_piece<SPLIT>(p, (int)(blockIdx.x % np), R.c_first, R.c_last);
  S.c_last = Pc.hi;
  S.io_k.init(p.ks[1]);
  S.io_v.init(p.vs[1]);
  q_prologue<T, D>(p, S.io_k, S.io_v, S.kbase, S.vbase, Pc.lo, Pc.hi, Ks, Vs);
  auto masked = [&](int c) { return c < R.cu0 || c > R.cu1; };
  int c = Pc.lo;
  for (; c + 2 <= Pc.hi; c += 3) {  // unrolled by three: compile-time LDS offsets
    dq_step<T, D, MODE, 0>(p, S, c, Ks, Vs, masked(c));
    dq_step<T, D, MODE, 1>(p, S, c + 1, Ks, Vs, masked(c + 1));
    dq_step<T, D, MODE, 2>(p, S, c + 2, Ks, Vs, masked(c + 2));
  }
  if (c <= Pc.hi) dq_step<T, D, MODE, 0>(p, S, c, Ks, Vs, masked(c));
  if (c + 1 <= Pc.hi) dq_step<T, D, MODE, 1>(p, S, c + 1, Ks, Vs, masked(c + 1));
  wait_vmem();  // the repeated loads of the last steps land before the workgroup ends

  if constexpr (SPLIT) {
    // this piece's unscaled partial dQ rows (fp32), merged by k_dq_merge
#pragma unroll
    for (int q = 0; q < NQB; ++q) {
      const int qi = S.qi[q];
      if (qi >= p.Sq) continue;
      float *wrow = p.ws_split + ((int64_t)Pc.piece * p.B * p.H * p.Sq +
                                  ((int64_t)b * p.H + h) * p.Sq + qi) * D;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4<float>(wrow + 32 * t + 8 * g + 4 * half, S.dq[q][t][4 * g], S.dq[q][t][4 * g + 1],
                        S.dq[q][t][4 * g + 2], S.dq[q][t][4 * g + 3]);
    }
    return;
  }
  const float sc = p.scale;  // the factor of dS, applied once
  typedef RowStore<T, D> RS;
  if constexpr (NQB == 1 && 4 * RS::BYTES <= sizeof(Ks)) {
    // whole rows through LDS (the chunk tiles are free once every wave is done)
    __syncthreads();
    char *lq = reinterpret_cast<char *>(Ks) + w * RS::BYTES;
    RS::write_tiles(S.dq[0], sc, lq, S.lane);
    const int q0 = i0 + 32 * w;
    T *dq0 = (T *)p.dq + b * p.dqs[0] + (int64_t)q0 * p.dqs[1] + h * p.dqs[2];
    RS::store_rows(lq, max(0, min(32, p.Sq - q0)), [&](int n) { return dq0 + (int64_t)n * p.dqs[1]; },
                   S.lane);
  } else {
#pragma unroll
    for (int q = 0; q < NQB; ++q) {
      const int qi = S.qi[q];
      if (qi >= p.Sq) continue;
      T *dqrow = (T *)p.dq + b * p.dqs[0] + (int64_t)qi * p.dqs[1] + h * p.dqs[2];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          store4<T>(dqrow + 32 * t + 8 * g + 4 * half, sc * S.dq[q][t][4 * g],
                    sc * S.dq[q][t][4 * g + 1], sc * S.dq[q][t][4 * g + 2],
                    sc * S.dq[q][t][4 * g + 3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Row statistics and dQ in one query-major pass (bf16): the chunk step and its
// arithmetic are sd_core.hpp's; here the chunks are 64 consecutive keys of the
// (b, h) head and the mask is the dense one.
template <typename T, int D> struct SdState {
  typedef MT<T> M;
  static constexpr int NSD = D / M::KS, NT = D / 32;
  typename M::frag qf[NSD], gf[NSD];
  f32x16 acc_a[NT], acc_b[NT];
  RowStat st;
  float dh;  // the estimate of delta that acc_a currently subtracts
  int qi;
  KeySpan ks;  // the keys the row sees by the index rule
  ChunkIO<T, D, kSdKeys> io_k, io_v;
  const T *kbase, *vbase;
  int b, h, lane, half, c_last;
};

// Chunk c (keys 64 c .. 64 c + 63), whose tiles are in buffer bc of four;
// chunk min(c + 2, c_last) goes to buffer bc + 2 (chunk c - 2's, whose phase C
// ran in step c - 1), one load per S step (past the end the last chunk is
// loaded again: never read, drained at the end).  With PREV, chunk c - 1's
// middle and phase C run in this step too (its K tile in buffer bc - 1).
template <typename T, int D, int MODE, bool MASKED, bool PREV>
__device__ __forceinline__ void sd_step(const DenseParams &p, SdState<T, D> &S, int c, int bc,
                                        Tile<T, D, kSdKeys> *Ks, Tile<T, D, kSdKeys> *Vs,
                                        SdCarry<T> &X) {
  constexpr int KC = kSdKeys, L = ChunkIO<T, D, KC>::LOADS;
  const int bn = (bc + 2) & 3, bp = (bc + 3) & 3;
  const int half = S.half, j0 = c * KC;
  const int cn = min(c + 2, S.c_last);
  const T *kn = S.kbase + (int64_t)cn * KC * p.ks[1];
  const T *vn = S.vbase + (int64_t)cn * KC * p.vs[1];
  const int lastn = p.Sk - 1 - cn * KC;
  const unsigned ksb = (unsigned)(p.ks[1] * sizeof(T)), vsb = (unsigned)(p.vs[1] * sizeof(T));
  constexpr unsigned TB = sizeof(Tile<T, D, KC>);
  const unsigned klds = lds_addr(Ks) + bn * TB, vlds = lds_addr(Vs) + bn * TB;
  auto dma = [&](int k) {
    if (k < L)
      S.io_k.issue_one_at(k, kn, lastn, ksb, klds);
    else
      S.io_v.issue_one_at(k - L, vn, lastn, vsb, vlds);
  };
  auto adj_of = [&](int u, int r) {
    return q_adj<MODE>(p, S.b, S.h, S.qi, j0 + 32 * u + kr(r, half), S.ks);
  };
  sd_body_deferred<T, D, MASKED, PREV>(S, p.scale_log2, &Ks[bc], &Vs[bc], &Ks[bp], X, adj_of, dma);
}


template <typename T, int D, int MODE, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_stats_dq(const DenseParams p) {
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NT = D / 32, QROWS = 128, KC = kSdKeys;
  static_assert(sizeof(T) == 2, "bf16 only (direct-to-LDS chunk loads)");
  static_assert(QShape<T>::QROWS == QROWS, "one 32-query block per wave");
  __shared__ Tile<T, D, KC> Ks[4], Vs[4];

  SdState<T, D> S;
  const int tid = threadIdx.x, w = tid >> 6;
  S.lane = tid & 63;
  S.half = S.lane >> 5;
  const int l32 = S.lane & 31, half = S.half;
  const int nb = p.nblk;
  int bh, rank;
  const int np = SPLIT ? p.npiece : 1;  // split form: consecutive workgroups are one block's pieces
  // the heaviest causal blocks first; under a narrow band the short first ones,
  // in groups of 8 heads (window-256: 76.8 -> 74.4 us against groups of
  // kDqGroup, with which the causal workload runs 1.5 us faster)
  const bool band = narrow_band(p);
  if (band)
    tile_order<8>(blockIdx.x / np, gridDim.x / np, nb, bh, rank);
  else
    tile_order<kDqGroup>(blockIdx.x / np, gridDim.x / np, nb, bh, rank);
  const int blk = band ? rank : nb - 1 - rank;
  S.h = bh % p.H;
  S.b = bh / p.H;
  const int b = S.b, h = S.h;
  const int i0 = blk * QROWS;
  {
    const int qi = i0 + 32 * w + l32;
    S.qi = qi;
    S.ks = key_span(p, qi);
    const bool qvalid = qi < p.Sq;
    const T *qrow = (const T *)p.q + b * p.qs[0] + (int64_t)(qvalid ? qi : 0) * p.qs[1] + h * p.qs[2];
    const T *grow = (const T *)p.dy + b * p.dys[0] + (int64_t)(qvalid ? qi : 0) * p.dys[1] + h * p.dys[2];
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      S.qf[s] = load_frag<T>(qrow, s * KS + half * KL, qvalid);
      S.gf[s] = load_frag<T>(grow, s * KS + half * KL, qvalid);
    }
    sd_init<NT>(S);
  }
  S.kbase = (const T *)p.k + b * p.ks[0] + (h / p.G) * p.ks[2];  // the head's K / V head
  S.vbase = (const T *)p.v + b * p.vs[0] + (h / p.G) * p.vs[2];
  const QRange R = q_range<KC>(p, i0, QROWS, MODE == MODE_INDEX);
  const QPiece Pc = q_piece<SPLIT>(p, (int)(blockIdx.x % np), R.c_first, R.c_last);
  S.c_last = Pc.hi;
  S.io_k.init(p.ks[1]);
  S.io_v.init(p.vs[1]);
  // Chunk c_first into buffer 0 and landed (with the fragment loads above);
  // chunk c_first + 1 into buffer 1 stays in flight under chunk c_first's
  // compute (the first step waits for it at its end, as for every chunk).
  if (Pc.lo <= Pc.hi) {
    S.io_k.issue(S.kbase, p.ks[1], Pc.lo * KC, p.Sk, Ks[0]);
    S.io_v.issue(S.vbase, p.vs[1], Pc.lo * KC, p.Sk, Vs[0]);
  }
  wait_vmem();
  __syncthreads();
  if (Pc.lo <= Pc.hi) {
    const int c1 = min(Pc.lo + 1, Pc.hi);
    S.io_k.issue(S.kbase, p.ks[1], c1 * KC, p.Sk, Ks[1]);
    S.io_v.issue(S.vbase, p.vs[1], c1 * KC, p.Sk, Vs[1]);
  }
  // Masked chunks before cu0 and after cu1, unmasked ones between (only for
  // the index rule with scale > 0: the unmasked step takes the max of the raw
  // scores); the buffers rotate at run time.
  int cu0 = R.cu0, cu1 = SPLIT ? min(R.cu1, Pc.hi) : R.cu1;
  if (!(p.scale_log2 > 0.f)) {
    cu0 = Pc.hi + 1;
    cu1 = Pc.hi;
  }
  int c = Pc.lo, bc = 0;
  auto next = [&]() {
    ++c;
    bc = (bc + 1) & 3;
  };
  SdCarry<T> X;
  if (c <= Pc.hi) {  // the first chunk has no pending one
    if (MODE == MODE_INDEX && c >= cu0 && c <= cu1)
      sd_step<T, D, MODE, false, false>(p, S, c, bc, Ks, Vs, X);
    else
      sd_step<T, D, MODE, true, false>(p, S, c, bc, Ks, Vs, X);
    next();
    for (; c < cu0 && c <= Pc.hi; next()) sd_step<T, D, MODE, true, true>(p, S, c, bc, Ks, Vs, X);
    if constexpr (MODE == MODE_INDEX)
      for (; c <= cu1; next()) sd_step<T, D, MODE, false, true>(p, S, c, bc, Ks, Vs, X);
    for (; c <= Pc.hi; next()) sd_step<T, D, MODE, true, true>(p, S, c, bc, Ks, Vs, X);
    sd_finish<T, D>(S, &Ks[(bc + 3) & 3], X);  // the last chunk's phase C
  }
  wait_vmem();  // the repeated loads of the last steps land before the workgroup ends

  if constexpr (SPLIT) {
    // This piece's partial results (merged by k_sdq_merge): per row (mref,
    // true max, l, delta', dh), then A' and B as whole rows through LDS (the
    // chunk tiles are free once every wave's repeated loads have landed).
    const int64_t rows = (int64_t)p.B * p.H * p.Sq;
    const int64_t row0 = ((int64_t)b * p.H + h) * p.Sq + i0 + 32 * w;  // the wave's first row
    const float l_tot = halves_sum(S.st.l);
    const float d_tot = halves_sum(S.st.dl);
    if (S.qi < p.Sq && half == 0) {
      float *r = p.ws_split + ((int64_t)Pc.piece * rows + row0 + l32) * 8;
      store4<float>(r, S.st.mref, S.st.mtrue, l_tot, d_tot);
      store4<float>(r + 4, S.dh, 0.f, 0.f, 0.f);
    }
    typedef RowStore<float, D> RSF;
    static_assert(2 * RSF::BYTES <= sizeof(Ks) && 2 * RSF::BYTES <= sizeof(Vs), "staging fits");
    __syncthreads();
    char *area = reinterpret_cast<char *>(w < 2 ? (void *)Ks : (void *)Vs) + (w & 1) * RSF::BYTES;
    const int nvalid = max(0, min(32, p.Sq - (i0 + 32 * w)));
    float *wa = p.ws_split + (int64_t)p.npiece * rows * 8 + ((int64_t)Pc.piece * rows + row0) * D;
    float *wb = wa + (int64_t)p.npiece * rows * D;
    RSF::write_tiles(S.acc_a, 1.f, area, S.lane);
    RSF::store_rows(area, nvalid, [&](int n) { return wa + (int64_t)n * D; }, S.lane);
    RSF::write_tiles(S.acc_b, 1.f, area, S.lane);  // LDS operations of a wave complete in order
    RSF::store_rows(area, nvalid, [&](int n) { return wb + (int64_t)n * D; }, S.lane);
    return;
  }

  const RowStatOut o = row_stat_final(S.st, p.inv_scale_log2);
  if (S.qi < p.Sq && half == 0) store_row_stat(p, ((int64_t)b * p.H + h) * p.Sq + S.qi, o);
  if (p.dq == nullptr) return;  // statistics only (dQ not requested)

  // dQ^T = A'^T * scale / l per lane column (row), once A' = A - dh B is moved
  // to A - delta B with delta = o.delta, the stored statistic.  Whole rows
  // stored through LDS: the chunk tiles are free once every wave's repeated
  // loads of the last step have landed (each wave waited for its own above;
  // the barrier covers the others').
  sd_settle<NT>(S, o.delta);
  __syncthreads();
  typedef RowStore<T, D> RS;
  static_assert(4 * RS::BYTES <= sizeof(Ks), "row staging fits the chunk tiles");
  char *lq = reinterpret_cast<char *>(Ks) + w * RS::BYTES;
  RS::write_tiles(S.acc_a, p.scale * o.inv_l, lq, S.lane);
  const int q0 = i0 + 32 * w;
  T *dq0 = (T *)p.dq + b * p.dqs[0] + (int64_t)q0 * p.dqs[1] + h * p.dqs[2];
  RS::store_rows(lq, max(0, min(32, p.Sq - q0)), [&](int n) { return dq0 + (int64_t)n * p.dqs[1]; },
                 S.lane);
}

// Merge of the split dK / dV: one thread per 4 columns of a key row, the
// pieces' accumulators added in piece order; dK = 0 - scale * sum (it was
// accumulated negated; a key no row sees gets +0), dV = sum.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_kv_merge(const DenseParams p) {
  const int64_t rows = (int64_t)p.B * p.Hkv * p.Sk;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tid >= rows * (D / 4)) return;
  const int dc = (int)(tid % (D / 4));
  const int64_t row = tid / (D / 4);
  const int j = (int)(row % p.Sk);
  const int64_t bg = row / p.Sk;
  const int g = (int)(bg % p.Hkv), b = (int)(bg / p.Hkv);
  f32x4 ak = {0.f, 0.f, 0.f, 0.f}, av = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < p.npiece; ++k) {
    const float *w = p.ws_split + (k * rows + row) * (2 * D) + 4 * dc;
    ak += *reinterpret_cast<const f32x4 *>(w);
    av += *reinterpret_cast<const f32x4 *>(w + D);
  }
  const float sc = p.scale;
  if (p.need_dk)
    store4<T>((T *)p.dk + b * p.dks[0] + (int64_t)j * p.dks[1] + g * p.dks[2] + 4 * dc,
              0.f - sc * ak[0], 0.f - sc * ak[1], 0.f - sc * ak[2], 0.f - sc * ak[3]);
  if (p.need_dv)
    store4<T>((T *)p.dv + b * p.dvs[0] + (int64_t)j * p.dvs[1] + g * p.dvs[2] + 4 * dc, av[0],
              av[1], av[2], av[3]);
}

// Merge of the split statistics + dQ pass (bf16): one thread per 4 columns of
// a row.  Pieces in order: the common reference M (largest mref), l = sum
// 2^(mref_k - M) l_k and delta' likewise, delta = delta' / l, and dQ = scale /
// l * sum 2^(mref_k - M) (A'_k + (dh_k - delta) B_k).  The row's first thread
// writes the statistics.  Partial layout: [npiece][rows][8] records, then
// [npiece][rows][D] of A', then of B.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_sdq_merge(const DenseParams p) {
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tid >= rows * (D / 4)) return;
  const int dc = (int)(tid % (D / 4));
  const int64_t row = tid / (D / 4);
  const int np = p.npiece;
  auto rec = [&](int k) { return p.ws_split + ((int64_t)k * rows + row) * 8; };
  float M = -INFINITY, mt = -INFINITY;
  for (int k = 0; k < np; ++k) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(rec(k));
    M = fmaxf(M, v[0]);
    mt = fmaxf(mt, v[1]);
  }
  float l = 0.f, dl = 0.f;
  if (M != -INFINITY) {
    for (int k = 0; k < np; ++k) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(rec(k));
      const float a = fast_exp2(v[0] - M);  // 0 for a piece that saw nothing
      l = fmaf(v[2], a, l);
      dl = fmaf(v[3], a, dl);
    }
  }
  const RowStatOut o = merged_row_stat(M, mt, l, dl, p.inv_scale_log2);
  if (dc == 0) store_row_stat(p, row, o);
  if (p.dq == nullptr) return;  // statistics only
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (!o.empty) {
    const float *abase = p.ws_split + (int64_t)np * rows * 8;
    const float *bbase = abase + (int64_t)np * rows * D;
    for (int k = 0; k < np; ++k) {
      const float *r = rec(k);
      if (r[0] == -INFINITY) continue;  // nothing seen in this piece
      const float a = fast_exp2(r[0] - M), sh = r[4] - o.delta;
      const f32x4 A = *reinterpret_cast<const f32x4 *>(abase + ((int64_t)k * rows + row) * D + 4 * dc);
      const f32x4 B = *reinterpret_cast<const f32x4 *>(bbase + ((int64_t)k * rows + row) * D + 4 * dc);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(a, fmaf(sh, B[e], A[e]), acc[e]);
    }
  }
  const int i = (int)(row % p.Sq);
  const int64_t bh = row / p.Sq;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const float sc = p.scale * o.inv_l;
  T *dst = (T *)p.dq + b * p.dqs[0] + (int64_t)i * p.dqs[1] + h * p.dqs[2] + 4 * dc;
  store4<T>(dst, sc * acc[0], sc * acc[1], sc * acc[2], sc * acc[3]);
}

// Merge of the split dQ: one thread per 4 columns of a row, the pieces' partial
// sums added in piece order, times `scale`, one store.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_dq_merge(const DenseParams p) {
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tid >= rows * (D / 4)) return;
  const int dc = (int)(tid % (D / 4));
  const int64_t row = tid / (D / 4);
  const int i = (int)(row % p.Sq);
  const int64_t bh = row / p.Sq;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < p.npiece; ++k)
    acc += *reinterpret_cast<const f32x4 *>(p.ws_split + (k * rows + row) * D + 4 * dc);
  const float sc = p.scale;
  T *dst = (T *)p.dq + b * p.dqs[0] + (int64_t)i * p.dqs[1] + h * p.dqs[2] + 4 * dc;
  store4<T>(dst, sc * acc[0], sc * acc[1], sc * acc[2], sc * acc[3]);
}

// ---------------------------------------------------------------------------
// Launchers: one instantiation per (element type, head dim, mask mode).

// Split form (p.ws_split set): nblocks * npiece workgroups, then the merge
// over the rows.
template <typename T, int D, int MODE>
static hipError_t launch_t(int stage, const DenseParams &p, int nblocks, hipStream_t stream) {
  const bool split = p.ws_split != nullptr;
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  if constexpr (sizeof(T) == 2) {
    if (split && stage == STAGE_STATS_DQ) {
      hipLaunchKernelGGL((k_stats_dq<T, D, MODE, true>), dim3(nblocks * p.npiece), dim3(256), 0,
                         stream, p);
      hipLaunchKernelGGL((k_sdq_merge<T, D>), dim3((unsigned)((rows * (D / 4) + 255) / 256)),
                         dim3(256), 0, stream, p);
      return hipGetLastError();
    }
  }
  if (split && stage == STAGE_KV) {
    const int64_t krows = (int64_t)p.B * p.Hkv * p.Sk;
    hipLaunchKernelGGL((k_kv_bwd<T, D, MODE, true>), dim3(nblocks * p.npiece), dim3(256), 0,
                       stream, p);
    hipLaunchKernelGGL((k_kv_merge<T, D>), dim3((unsigned)((krows * (D / 4) + 255) / 256)),
                       dim3(256), 0, stream, p);
  } else if (split && stage == STAGE_ROW_STATS) {
    hipLaunchKernelGGL((k_row_stats<T, D, MODE, true>), dim3(nblocks * p.npiece), dim3(256), 0,
                       stream, p);
    hipLaunchKernelGGL(k_rs_merge, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, p);
  } else if (split) {
    hipLaunchKernelGGL((k_dq_bwd<T, D, MODE, true>), dim3(nblocks * p.npiece), dim3(256), 0,
                       stream, p);
    hipLaunchKernelGGL((k_dq_merge<T, D>), dim3((unsigned)((rows * (D / 4) + 255) / 256)),
                       dim3(256), 0, stream, p);
  } else if (stage == STAGE_ROW_STATS)
    hipLaunchKernelGGL((k_row_stats<T, D, MODE, false>), dim3(nblocks), dim3(256), 0, stream, p);
  else if (stage == STAGE_KV)
    hipLaunchKernelGGL((k_kv_bwd<T, D, MODE, false>), dim3(nblocks), dim3(256), 0, stream, p);
  else if (stage == STAGE_DQ)
    hipLaunchKernelGGL((k_dq_bwd<T, D, MODE, false>), dim3(nblocks), dim3(256), 0, stream, p);
  else if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((k_stats_dq<T, D, MODE, false>), dim3(nblocks), dim3(256), 0, stream, p);
  else
    return hipErrorInvalidValue;  // the fused pass is built for bf16 only
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
