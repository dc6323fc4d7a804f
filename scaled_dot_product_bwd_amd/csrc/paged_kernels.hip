// paged_kernels.hip -- the gfx950 kernel of the paged, grouped-query history
// backward (dK / dV only), ruDNN 0.1.43 src/paged_attention/ordered_kernel.rs
// `history_backward`.
//
// The pages give one wavefront to each (physical token, KV head), which walks
// the page's links, the linked sequence's query rows and the group's query
// heads, forms each score with a cross-lane dot product and accumulates
// dK += ds q, dV += p dY, then stores once.  The same contraction over a whole
// item of 128 slots is dense enough for MFMA: one workgroup per (item, KV head
// g), 4 waves of 32 slots each (slot = MFMA column, K / V rows in registers),
// and the linked sequence's query rows times the group's query heads as the
// streamed row dimension ("qh rows", 64 per chunk for bf16).  Per chunk the
// body is the dense kernel's (kv_core.hpp); what differs is the addressing:
//   * qh row -> (row, head) and the row's position come from the plan
//     (rowinfo, fetched two chunks ahead of the Q / dY rows it addresses);
//   * P uses the supplied statistics, lse2 = max * log2 e + log2(denominator)
//     (a zero denominator gives P = 0, as the pages skip such rows);
//   * slot t of the item is visible to row r iff its token in the linked
//     sequence exists and, when causal, is <= the row's position.
// Each (slot, KV head) element is stored exactly once after all links: the
// gradient, or +0 for a slot no link reaches (tail slots, whose K / V rows are
// never read).  Slots of pages no sequence lists are never touched.
//
// Latent variant (the pages' `mla` switch): a slot holds one latent row c of
// width D that is both key and value, plus a position key of width P; a query
// row holds q (width D) and qp (width P).  The score contracts [q | qp] with
// [c | kp] (width D + P), dP contracts dY with c, and the latent receives both
// derivatives, d c = scale dS^T q + P^T dY, while the position key gets
// scale dS^T qp.  The body is the same with key width D + P and value width D:
// the V fragments are the first D / KS key fragments, dK's last P / 32 tiles
// are the position-key gradient, and the latent's two parts are summed at the
// store.
#include <atomic>
#include <type_traits>

#include "device_common.hpp"
#include "kv_core.hpp"
#include "paged.hpp"

namespace attn {

// Per-wave LDS copies of the row metadata.  Stats buffer (one per chunk in
// flight): m -> lse2, den, delta, position; 64 entries each (fp32 chunks use
// the first 32).  Rowinfo buffer: rh of the chunk's qh rows.
constexpr int kStatWave = 4 * 64;
constexpr int kStatWords = 4 * kStatWave;
constexpr int kRiWords = 4 * 64;

// D: value / latent width; P: position-key width (latent variant only, else 0).
// A latent wider than 128 takes 32-row chunks (its Q / dY tiles are wide).
template <typename T_, int D_, int P_, bool MLA_> struct PagedState {
  typedef T_ T;
  typedef MT<T> M;
  static constexpr int D = D_, P = P_, DK = D_ + P_;
  static constexpr bool MLA = MLA_;
  static constexpr int NSD = DK / M::KS, NSV = D / M::KS, NT = DK / 32, NTV = D / 32;
  static constexpr int ROWS = (MLA && D > 128) ? 32 : KvShape<T>::ROWS;
  typedef Tile<T, DK, ROWS> QTile;  // Q rows (latent variant: [q | qp])
  typedef Tile<T, D, ROWS> GTile;   // dY rows
  typename M::frag kf[NSD], vf[MLA ? 1 : NSV];
  f32x16 dk[NT], dv[MLA ? 1 : NTV];  // latent variant: dk holds both derivatives
  ChunkIO<T, DK, ROWS> io_q;
  ChunkIO<T, D, ROWS> io_g;
  const T *qbase, *qpbase, *gbase;  // Q / qp / dY at head g * group
  const float *sbase;               // statistics at head g * group
  const int32_t *rh_tab, *pos_tab;  // the link's sequence: qh rows from 0
  int nqh, c_last, tok, wave, lane, buf;
};

// A processed link of a (item, KV head) unit, as read from its plan record
// (all fields wave-uniform).  k: the unit's place in the workgroup's list,
// -1 for "no more".
struct PagedSeg {
  int k, g, item, li, qh0, nqh, masked;
};

// A plan word at a wave-uniform index, read through the constant address
// space: the plan does not change during a kernel, so this is a scalar load,
// waited on by itself (not behind the vector loads in flight).
__device__ __forceinline__ int plan_word(const int32_t *plan, int64_t idx) {
  typedef __attribute__((address_space(4))) const int32_t cint;
  return ((cint *)(uintptr_t)plan)[idx];
}

// Rowinfo of chunk c of the nqh qh rows at rh_tab into the buffer at LDS byte
// address ri_lds (an integer, so a buffer picked at run time costs no
// generic-pointer arithmetic): lane l <- rh of row c * ROWS + l, clamped to the
// last row so every lane reads inside the plan.
template <typename St>
__device__ __forceinline__ void issue_rows_at(const St &S, const int32_t *rh_tab, int nqh, int c,
                                              unsigned ri_lds) {
  const int qh = min(c * St::ROWS + S.lane, nqh - 1);
  dma_lds4_at(__builtin_amdgcn_readfirstlane(ri_lds + 4u * 64 * S.wave), rh_tab + qh);
}
template <typename St>
__device__ __forceinline__ void issue_rowinfo_at(St &S, int c, unsigned ri_lds) {
  issue_rows_at(S, S.rh_tab, S.nqh, c, ri_lds);
}
template <typename St>
__device__ __forceinline__ void issue_rowinfo(St &S, int c, int *ri) {
  issue_rowinfo_at(S, c, lds_addr(ri));
}

// Where a link's rows live: Q / dY / statistics at head g * group of the
// link's KV head, and its qh rows' row ids and positions.
template <typename T> struct LinkRows {
  const T *qbase, *qpbase, *gbase;
  const float *sbase;
  const int32_t *rh_tab, *pos_tab;
  int nqh;
};

// Statistics and Q / dY rows of chunk c of link L; `ri` holds the chunk's
// rowinfo (landed).  With direct-to-LDS loads the buffers are addressed by
// their LDS byte addresses (integers: st_lds, q_lds, g_lds); register-staged
// loads (fp32) go through the tile pointers.  Issues 4 + the tiles' loads.
template <typename St>
__device__ __forceinline__ void issue_chunk_of(const PagedParams &p, St &S,
                                               const LinkRows<typename St::T> &L, int c,
                                               const int *ri, unsigned st_lds,
                                               typename St::QTile *Q, typename St::GTile *G,
                                               unsigned q_lds, unsigned g_lds) {
  typedef typename St::T T;
  constexpr int D = St::D, P = St::P;
  const int *myri = ri + 64 * S.wave;
  const unsigned myst = __builtin_amdgcn_readfirstlane(st_lds + 4u * kStatWave * S.wave);
  const int rh = myri[S.lane];
  const float *srow = L.sbase + 3 * (int64_t)rh;
  dma_lds4_at(myst, srow);
  dma_lds4_at(myst + 4u * 64, srow + 1);
  dma_lds4_at(myst + 4u * 128, srow + 2);
  dma_lds4_at(myst + 4u * 192, L.pos_tab + min(c * St::ROWS + S.lane, L.nqh - 1));
  auto qelem = [&](int r, int col) {
    if constexpr (P > 0)  // a row of the tile is [q | qp]: columns below D from q, the rest from qp
      return col < D ? L.qbase + (int64_t)myri[r] * D + col
                     : L.qpbase + (int64_t)myri[r] * P + (col - D);
    else
      return L.qbase + (int64_t)myri[r] * D + col;
  };
  auto gelem = [&](int r, int col) { return L.gbase + (int64_t)myri[r] * D + col; };
  if constexpr (ChunkIO<T, St::DK, St::ROWS>::DIRECT) {
    S.io_q.issue_elem_at(qelem, q_lds);
    S.io_g.issue_elem_at(gelem, g_lds);
  } else {
    S.io_q.issue_elem(qelem, *Q);
    S.io_g.issue_elem(gelem, *G);
  }
}
// The same for the state's current link.
template <typename St>
__device__ __forceinline__ void issue_chunk(const PagedParams &p, St &S, int c, const int *ri,
                                            unsigned st_lds, typename St::QTile *Q,
                                            typename St::GTile *G, unsigned q_lds,
                                            unsigned g_lds) {
  const LinkRows<typename St::T> L{S.qbase, S.qpbase, S.gbase, S.sbase, S.rh_tab, S.pos_tab, S.nqh};
  issue_chunk_of(p, S, L, c, ri, st_lds, Q, G, q_lds, g_lds);
}
template <typename St>
__device__ __forceinline__ void issue_chunk(const PagedParams &p, St &S, int c, const int *ri,
                                            float *st, typename St::QTile *Q,
                                            typename St::GTile *G) {
  issue_chunk(p, S, c, ri, lds_addr(st), Q, G, lds_addr(Q), lds_addr(G));
}

// Replace max by -lse2 / scale_log2 in this wave's statistics of chunk c
// (landed): the kv body's starting score.  Rows past the sequence's last qh
// row get -inf, so P = 0 for them with or without the per-element test.
template <typename St>
__device__ __forceinline__ void convert_stats(const PagedParams &p, St &S, int c, float *st) {
  float *myst = st + kStatWave * S.wave;
  const int l = S.lane;
  const bool real = l < St::ROWS && c * St::ROWS + l < S.nqh;
  const float m = myst[l], den = myst[64 + l];
  myst[l] = ((real && den > 0.f) ? -fmaf(m, kLog2e, log2f(den)) : -INFINITY) * p.inv_scale_log2;
}

// Convert and consume chunk c of the state's link (landed; its statistics at
// st, tiles Q, G): the kv body (MASKED: per-element visibility).
template <bool MASKED, typename St>
__device__ __forceinline__ void consume_chunk(const PagedParams &p, St &S, int c, float *st,
                                              typename St::QTile *Q, typename St::GTile *G) {
  typedef typename St::T T;
  convert_stats(p, S, c, st);
  const float *myst = st + kStatWave * S.wave;
  const int *posv = reinterpret_cast<const int *>(myst + 192);
  const int tok = S.tok, half = S.lane >> 5;
  const bool causal = p.causal;
  // Slot visible to the row: its token exists and, when causal, is <= the
  // position (non-short-circuit operators: one LDS read and no branch per element).
  auto adj = [&](int u, int r) -> float {
    const int pos = posv[32 * u + kr(r, half)];
    const bool vis = (tok >= 0) & (!causal | (tok <= pos));
    return vis ? 0.f : -INFINITY;
  };
  kv_chunk<T, St::DK, St::D, MASKED, St::MLA, 0, decltype(adj), NoDma, false, St::ROWS / 32>(
      S.kf, St::MLA ? S.kf : S.vf, S.dk, S.dv, Q, G, myst, myst + 128, p.scale_log2, S.lane, adj,
      p.scale);
}

// One chunk: request rowinfo of chunk c + 4 and the data of chunk c + 2,
// consume chunk c, hand over.  Chunk k's tiles, statistics and rowinfo sit in
// buffer k % 3 (S.buf = c % 3).
template <bool MASKED, typename St>
__device__ __forceinline__ void paged_step(const PagedParams &p, St &S, int c,
                                           typename St::QTile *Qs, typename St::GTile *Gs,
                                           float (*st)[kStatWords], int (*ri)[kRiWords]) {
  typedef typename St::T T;
  constexpr int PER_CHUNK =
      5 + ChunkIO<T, St::DK, St::ROWS>::LOADS + ChunkIO<T, St::D, St::ROWS>::LOADS;
  static_assert(PER_CHUNK < 64, "vmcnt budget");
  const int bc = S.buf, bn = bc == 0 ? 2 : bc - 1, bz = bc == 2 ? 0 : bc + 1;
  const bool issued = c + 2 <= S.c_last;
  if (issued) {
    // LDS byte addresses of the run-time-picked buffers, as wave-uniform integers
    constexpr unsigned QB = sizeof(Qs[0]), GB = sizeof(Gs[0]), SB = sizeof(st[0]),
                       RB = sizeof(ri[0]);
    auto uni = [](unsigned x) { return (unsigned)__builtin_amdgcn_readfirstlane(x); };
    issue_rowinfo_at(S, c + 4, uni(lds_addr(ri) + bz * RB));  // always issued with the chunk
    issue_chunk(p, S, c + 2, ri[bn], uni(lds_addr(st) + bn * SB), &Qs[bn], &Gs[bn],
                uni(lds_addr(Qs) + bn * QB), uni(lds_addr(Gs) + bn * GB));
  }
  consume_chunk<MASKED>(p, S, c, st[bc], &Qs[bc], &Gs[bc]);
  if (issued) {
    S.io_q.complete(Qs[bn]);
    S.io_g.complete(Gs[bn]);
  }
  if constexpr (ChunkIO<T, St::D, St::ROWS>::DIRECT) {
    if (issued)
      wait_vmem_le<PER_CHUNK>();
    else
      wait_vmem();
  } else {
    wait_vmem();
  }
  __syncthreads();
  S.buf = bz;
}

// The first two chunks of a link: their data (rowinfo of chunks 0 .. 2
// already landed in ri[0 .. 2]) and the rowinfo of chunk 3; mid() runs while
// those loads are in flight; then everything lands and the workgroup
// synchronises.
template <typename St, typename Mid>
__device__ __forceinline__ void paged_prologue(const PagedParams &p, St &S, typename St::QTile *Qs,
                                               typename St::GTile *Gs, float (*st)[kStatWords],
                                               int (*ri)[kRiWords], Mid mid) {
  issue_chunk(p, S, 0, ri[0], st[0], &Qs[0], &Gs[0]);
  S.io_q.complete(Qs[0]);
  S.io_g.complete(Gs[0]);
  if (S.c_last >= 1) {
    issue_chunk(p, S, 1, ri[1], st[1], &Qs[1], &Gs[1]);
    S.io_q.complete(Qs[1]);
    S.io_g.complete(Gs[1]);
  }
  issue_rowinfo(S, 3, ri[0]);
  mid();
  wait_vmem();
  __syncthreads();
  S.buf = 0;
}

// The chunk loop of one link (rowinfo of chunk k fetched at step k - 4, read at
// step k - 2).  The link runs the unmasked body when every lane holds a token
// that every row of the sequence sees; otherwise the masked one.  Each variant
// has its own loop.
template <typename St>
__device__ __forceinline__ void paged_chunks(const PagedParams &p, St &S, bool masked,
                                             typename St::QTile *Qs, typename St::GTile *Gs,
                                             float (*st)[kStatWords], int (*ri)[kRiWords]) {
  const int c_last = S.c_last;
  if (masked) {
    for (int c = 0; c <= c_last; ++c) paged_step<true>(p, S, c, Qs, Gs, st, ri);
  } else {
    for (int c = 0; c <= c_last; ++c) paged_step<false>(p, S, c, Qs, Gs, st, ri);
  }
}

// The link's tables and counts into the state (qh0, nqh: its record's first
// qh row and qh row count).
template <typename St>
__device__ __forceinline__ void begin_link(const PagedParams &p, St &S, int qh0, int nqh) {
  S.nqh = nqh;
  S.rh_tab = p.plan + p.off_qh_rh + qh0;
  S.pos_tab = p.plan + p.off_qh_pos + qh0;
  S.c_last = (nqh - 1) / St::ROWS;
}

// A link's plan record, read with scalar loads.
struct LinkRec {
  int min_tok, max_tok, all_valid, qh0, nqh, minpos, maxpos;
  __device__ __forceinline__ LinkRec(const PagedParams &p, int li) {
    const int64_t o = p.off_link_info + (int64_t)plan::LINK_INFO_WORDS * li;
    min_tok = plan_word(p.plan, o + plan::LI_MIN_TOK);
    max_tok = plan_word(p.plan, o + plan::LI_MAX_TOK);
    all_valid = plan_word(p.plan, o + plan::LI_ALL_VALID);
    qh0 = plan_word(p.plan, o + plan::LI_QH0);
    nqh = plan_word(p.plan, o + plan::LI_NQH);
    minpos = plan_word(p.plan, o + plan::LI_MINPOS);
    maxpos = plan_word(p.plan, o + plan::LI_MAXPOS);
  }
  // Processed: the sequence has query rows and, when causal, some row can see
  // one of the item's tokens.
  __device__ __forceinline__ bool processed(bool causal) const {
    return nqh > 0 && !(causal && min_tok > maxpos);
  }
  // Masked body needed: not every lane holds a token that every row sees.
  __device__ __forceinline__ bool masked(bool causal) const {
    return !(all_valid != 0 && (!causal || minpos >= max_tok));
  }
};

// The wave's K / V (latent variant: latent and position key) fragments of the
// pool rows the slot entry `ent` names (zero for a lane without a live slot).
// The loads go straight into the fragment registers, so they are all in flight
// together.
template <typename St>
__device__ __forceinline__ void load_kv(const PagedParams &p, St &S, int ent, int g) {
  typedef typename St::T T;
  constexpr int D = St::D, P = St::P, KS = St::M::KS, KL = St::M::KL;
  const int half = S.lane >> 5;
  const bool live = ent >= 0 && (ent & 1);
  const int64_t srow = (int64_t)(ent >= 0 ? ent >> 1 : 0) * p.kv_heads + g;  // pool row
  const T *krow = (const T *)p.k_pool + srow * D;
  const T *kprow = (const T *)p.kp_pool + srow * P;
#pragma unroll
  for (int s = 0; s < St::NSD; ++s) {
    // fragment s covers columns s * KS .. s * KS + KS - 1: the key's when
    // below D, else the position key's (KS divides D)
    if (s * KS < D)
      S.kf[s] = load_frag<T>(krow, s * KS + half * KL, live);
    else
      S.kf[s] = load_frag<T>(kprow, s * KS - D + half * KL, live);
  }
  if constexpr (!St::MLA) {
    const T *vrow = (const T *)p.v_pool + srow * D;
#pragma unroll
    for (int s = 0; s < St::NSV; ++s) S.vf[s] = load_frag<T>(vrow, s * KS + half * KL, live);
  }
}

template <typename St> __device__ __forceinline__ void zero_acc(St &S) {
#pragma unroll
  for (int t = 0; t < St::NT; ++t) S.dk[t] = f32x16{};
#pragma unroll
  for (int t = 0; t < (St::MLA ? 1 : St::NTV); ++t) S.dv[t] = f32x16{};
}

// One store per (slot, KV head) element of the unit (slot entry `ent` in each
// lane, KV head g): the gradient, +0 for a tail slot; lanes without a slot
// store nothing.  Whole rows go through this wave's part of the tile buffers
// (every wave must be done with them): every lane stores 16 contiguous bytes.
template <typename St>
__device__ __forceinline__ void store_unit_rows(const PagedParams &p, St &S, int ent, int g,
                                                char *qbuf, char *gbuf) {
  typedef typename St::T T;
  constexpr int D = St::D, P = St::P;
  typedef RowStore<T, D> RSd;
  typedef RowStore<T, (P > 0 ? P : 32)> RSp;
  const int lane = fresh(S.lane);
  const bool live = ent >= 0 && (ent & 1);
  const float sc = live ? p.scale : 0.f;  // dS's factor, applied once; tails store +0
  char *l0 = qbuf + S.wave * RSd::BYTES;
  char *lp = qbuf + 4 * RSd::BYTES + S.wave * RSp::BYTES;
  char *l1 = gbuf + S.wave * RSd::BYTES;
  // pool row of the wave's slot n (lane n holds its entry), -1 for no slot
  auto row_of = [&](int n) -> int64_t {
    const int e = __shfl(ent, n);
    return e < 0 ? -1 : (int64_t)(e >> 1) * p.kv_heads + g;
  };
  if constexpr (St::MLA) {
    // dk holds both derivatives already scaled: the latent's tiles, then the position key's
    if (p.need_dk) RSd::write_tiles(S.dk, live ? 1.f : 0.f, l0, lane);
    if (P > 0 && p.need_dkp) RSp::write_tiles(S.dk + D / 32, live ? 1.f : 0.f, lp, lane);
    if (p.need_dk)
      RSd::store_rows(l0, 32, [&](int n) -> T * {
        const int64_t r = row_of(n);
        return r < 0 ? nullptr : (T *)p.dk_pool + r * D;
      }, lane);
    if (P > 0 && p.need_dkp)
      RSp::store_rows(lp, 32, [&](int n) -> T * {
        const int64_t r = row_of(n);
        return r < 0 ? nullptr : (T *)p.dkp_pool + r * P;
      }, lane);
  } else {
    if (p.need_dk) RSd::write_tiles(S.dk, sc, l0, lane);
    if (p.need_dv) RSd::write_tiles(S.dv, live ? 1.f : 0.f, l1, lane);
    if (p.need_dk)
      RSd::store_rows(l0, 32, [&](int n) -> T * {
        const int64_t r = row_of(n);
        return r < 0 ? nullptr : (T *)p.dk_pool + r * D;
      }, lane);
    if (p.need_dv)
      RSd::store_rows(l1, 32, [&](int n) -> T * {
        const int64_t r = row_of(n);
        return r < 0 ? nullptr : (T *)p.dv_pool + r * D;
      }, lane);
  }
}

// The same for the persistent form (not latent) through one area of
// RowStore<T, D>::BYTES per wave: dK's rows, then dV's over them.  Batched so
// that a wave waits on LDS a few times, not once per row: the slot entries of
// all the lane's store rows first (ents: the wave's 32 entries in LDS), then
// per matrix all tile writes, all row reads, all stores.  LDS operations of a
// wave complete in order, so dV's writes follow dK's reads.
template <typename St>
__device__ __forceinline__ void store_unit_rows_seq(const PagedParams &p, St &S, int ent,
                                                    const int *ents, int g, char *area) {
  typedef typename St::T T;
  constexpr int D = St::D;
  typedef RowStore<T, D> RS;
  constexpr int NIT = 32 / RS::RPI;  // store instructions per matrix
  const int lane = fresh(S.lane), c = lane % RS::LPR;
  const bool live = ent >= 0 && (ent & 1);
  int64_t row[NIT];  // element offset of the lane's row n = it * RPI + lane / LPR, -1 for no slot
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int e = ents[it * RS::RPI + lane / RS::LPR];
    row[it] = e < 0 ? -1 : ((int64_t)(e >> 1) * p.kv_heads + g) * D;
  }
  auto put = [&](const f32x16 *acc, float scale, T *pool) {
    RS::write_tiles(acc, scale, area, lane);
    f32x4 x[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it)
      x[it] = *reinterpret_cast<const f32x4 *>(area + (it * RS::RPI + lane / RS::LPR) * RS::RB + 16 * c);
#pragma unroll
    for (int it = 0; it < NIT; ++it)
      if (row[it] >= 0)
        *reinterpret_cast<f32x4 *>(reinterpret_cast<char *>(pool + row[it]) + 16 * c) = x[it];
  };
  if (p.need_dk) put(S.dk, live ? p.scale : 0.f, (T *)p.dk_pool);  // dS's factor, applied once
  if (p.need_dv) put(S.dv, live ? 1.f : 0.f, (T *)p.dv_pool);
}

template <typename T, int D, int P, bool MLA>
__global__ __launch_bounds__(256) void k_paged_kv_bwd(const PagedParams p) {
  typedef PagedState<T, D, P, MLA> St;
  __shared__ typename St::QTile Qs[3];
  __shared__ typename St::GTile Gs[3];
  __shared__ __attribute__((aligned(16))) float st[3][kStatWords];
  __shared__ __attribute__((aligned(16))) int ri[3][kRiWords];

  St S;
  S.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  S.lane = threadIdx.x & 63;
  const int l32 = S.lane & 31, half = S.lane >> 5;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int g = L / p.items, item = L % p.items;  // consecutive ids: one KV head, adjacent items
  const int32_t *plan = p.plan;

  const int ent = plan[p.off_item_slots + item * plan::kItemSlots + 32 * S.wave + l32];
  const bool live = ent >= 0 && (ent & 1);
  const int64_t srow = (int64_t)(ent >= 0 ? ent >> 1 : 0) * p.kv_heads + g;  // pool row
  load_kv(p, S, ent, g);
  zero_acc(S);
  S.io_q.init(St::DK);
  S.io_g.init(D);
  const int hg = g * p.group;
  S.qbase = (const T *)p.q + (int64_t)hg * D;
  S.qpbase = (const T *)p.qp + (int64_t)hg * P;
  S.gbase = (const T *)p.dy + (int64_t)hg * D;
  S.sbase = p.stats + 3 * (int64_t)hg;

  const int lb = plan_word(plan, p.off_item_links + item);
  const int le = plan_word(plan, p.off_item_links + item + 1);
  for (int li = lb; li < le; ++li) {
    const LinkRec rec(p, li);
    if (!rec.processed(p.causal)) continue;  // no rows, or no row sees the item
    begin_link(p, S, rec.qh0, rec.nqh);
    S.tok = plan[p.off_link_tok + li * plan::kItemSlots + 32 * S.wave + l32];
    const bool masked = rec.masked(p.causal);
    issue_rowinfo(S, 0, ri[0]);
    issue_rowinfo(S, 1, ri[1]);
    issue_rowinfo(S, 2, ri[2]);
    wait_vmem();
    paged_prologue(p, S, Qs, Gs, st, ri, [] {});
    paged_chunks(p, S, masked, Qs, Gs, st, ri);
  }

  // One store per (slot, KV head) element: the gradient, +0 for a tail slot;
  // unused lanes (no slot) store nothing.  Whole rows through LDS when the
  // staging fits the chunk tiles (free once every wave is done).
  typedef RowStore<T, D> RSd;
  typedef RowStore<T, (P > 0 ? P : 32)> RSp;
  if constexpr (4 * (RSd::BYTES + (MLA && P > 0 ? RSp::BYTES : 0)) <= sizeof(Qs) &&
                4 * RSd::BYTES <= sizeof(Gs)) {
    __syncthreads();
    store_unit_rows(p, S, ent, g, reinterpret_cast<char *>(Qs), reinterpret_cast<char *>(Gs));
    return;
  }
  const float sc = live ? p.scale : 0.f;  // dS's factor, applied once; tails store +0
  if (ent < 0) return;
  if constexpr (MLA) {
    // dS was scaled before its products: dk holds the latent's gradient (both
    // derivatives) and then the position key's; tails store +0
    T *dcrow = (T *)p.dk_pool + srow * D;
    T *dprow = (T *)p.dkp_pool + srow * P;
#pragma unroll
    for (int t = 0; t < St::NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d0 = 32 * t + 8 * q + 4 * half;
        const f32x16 &a = S.dk[t];
        T *dst = t < St::NTV ? (p.need_dk ? dcrow + d0 : nullptr)
                             : (p.need_dkp ? dprow + (d0 - D) : nullptr);
        if (dst)
          store4<T>(dst, live ? a[4 * q] : 0.f, live ? a[4 * q + 1] : 0.f,
                    live ? a[4 * q + 2] : 0.f, live ? a[4 * q + 3] : 0.f);
      }
  } else {
    T *dkrow = (T *)p.dk_pool + srow * D;
    T *dvrow = (T *)p.dv_pool + srow * D;
#pragma unroll
    for (int t = 0; t < St::NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d0 = 32 * t + 8 * q + 4 * half;
        const f32x16 &a = S.dk[t], &b = S.dv[t];
        if (p.need_dk)
          store4<T>(dkrow + d0, sc * a[4 * q], sc * a[4 * q + 1], sc * a[4 * q + 2], sc * a[4 * q + 3]);
        if (p.need_dv)
          store4<T>(dvrow + d0, live ? b[4 * q] : 0.f, live ? b[4 * q + 1] : 0.f,
                    live ? b[4 * q + 2] : 0.f, live ? b[4 * q + 3] : 0.f);
      }
  }
}

// ---------------------------------------------------------------------------
// Persistent form.
//
// The (item, KV head) units keep the classic form's order: unit L = g * items
// + item, each XCD owning a contiguous range of L (so adjacent items of one KV
// head, which share their sequences' Q / dY rows, run together in one L2).
// Workgroup j of an XCD takes the range's units j, j + W, j + 2 W, ... (W
// workgroups per XCD).  Within a unit the processed links run in plan order,
// exactly as in the classic form, so both forms give identical bits.
struct PagedUnits {
  int ub, j, per, cnt;  // the XCD's first unit, this workgroup's place, workgroups / units per XCD
  __device__ __forceinline__ int count() const { return j < cnt ? (cnt - j + per - 1) / per : 0; }
  __device__ __forceinline__ int unit(int k) const { return ub + j + k * per; }
};

// Zero gradients for every slot of a unit whose links are all skipped (no
// rows, or no row sees the item): what the classic form stores for it (its
// accumulators stay 0).  Rare; plain stores straight from registers.
template <typename St>
__device__ __forceinline__ void zero_unit(const PagedParams &p, const St &S, int item, int g) {
  typedef typename St::T T;
  constexpr int D = St::D;
  const int lane = fresh(S.lane), l32 = lane & 31, half = lane >> 5;
  const int e = p.plan[p.off_item_slots + item * plan::kItemSlots + 32 * S.wave + l32];
  if (e < 0) return;
  const int64_t srow = (int64_t)(e >> 1) * p.kv_heads + g;
  const float zk = (e & 1) ? p.scale * 0.f : 0.f;  // as the classic form: scale times a zero sum
  T *dkrow = (T *)p.dk_pool + srow * D;
  T *dvrow = (T *)p.dv_pool + srow * D;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d0 = 32 * t + 8 * q + 4 * half;
      if (p.need_dk) store4<T>(dkrow + d0, zk, zk, zk, zk);
      if (p.need_dv) store4<T>(dvrow + d0, 0.f, 0.f, 0.f, 0.f);
    }
}

// The first processed link at or after link li0 of unit k (li0 < 0: from the
// unit's first link), moving on to later units; a unit none of whose links is
// processed gets its zero stores on the way.
template <typename St>
__device__ __forceinline__ PagedSeg find_seg(const PagedParams &p, const St &S,
                                             const PagedUnits &W, int k, int li0) {
  const int32_t *plan = p.plan;
  const int n = W.count();
  PagedSeg s = {-1, 0, 0, 0, 0, 1, 0};
  for (; k < n; ++k, li0 = -1) {
    const int L = W.unit(k);
    const int g = L / p.items, item = L % p.items;
    const int lb = plan_word(plan, p.off_item_links + item);
    const int le = plan_word(plan, p.off_item_links + item + 1);
    for (int li = li0 < 0 ? lb : li0; li < le; ++li) {
      const LinkRec rec(p, li);
      if (!rec.processed(p.causal)) continue;
      s.k = k;
      s.g = g;
      s.item = item;
      s.li = li;
      s.qh0 = rec.qh0;
      s.nqh = rec.nqh;
      s.masked = rec.masked(p.causal);
      return s;
    }
    if (li0 < 0) zero_unit(p, S, item, g);
  }
  return s;
}

// vmcnt wait for a count known only at run time: n is one of the counts a
// persistent step leaves in flight (PD: a chunk's data loads, PC: with its
// rowinfo load); anything else waits for everything.
template <int PD, int PC>
__device__ __forceinline__ void wait_vmem_upto(int n) {
  if (n == PC)
    wait_vmem_le<PC>();
  else if (n == PD)
    wait_vmem_le<PD>();
  else
    wait_vmem();
}

template <int D>
__global__ __launch_bounds__(256) void k_paged_kv_persist(const PagedParams p) {
  typedef bf16 T;
  typedef PagedState<T, D, 0, false> St;
  constexpr int ROWS = St::ROWS;
  // loads of one chunk's data (statistics, positions, Q / dY tiles), and with
  // its rowinfo load
  constexpr int PD = 4 + ChunkIO<T, D, ROWS>::LOADS + ChunkIO<T, D, ROWS>::LOADS;
  constexpr int PC = PD + 1;
  static_assert(PC < 64, "vmcnt budget");
  __shared__ typename St::QTile Qs[3];
  __shared__ typename St::GTile Gs[3];
  __shared__ __attribute__((aligned(16))) float st[3][kStatWords];
  // Rowinfo banks: bank = link parity, slot = chunk % 4; a link's chunks 0 .. 3
  // are fetched into its bank while the previous link runs.
  __shared__ __attribute__((aligned(16))) int rib[2][4][kRiWords];
  // Per wave and lane: the current unit's slot entry, the next link's token
  // and the next unit's slot entry (fetched ahead, read at the switch).
  __shared__ __attribute__((aligned(16))) int ahead[3][4 * 64];
  // A finished unit's rows are staged in the buffer of its last chunk (waves
  // 0, 1 in its Q tile, waves 2, 3 in its dY tile) while the next link's first
  // two chunks sit in the other two.
  static_assert(2 * RowStore<T, D>::BYTES <= sizeof(Qs[0]) &&
                    2 * RowStore<T, D>::BYTES <= sizeof(Gs[0]),
                "row staging fits one buffer");

  St S;
  S.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  S.lane = threadIdx.x & 63;
  const int32_t *plan = p.plan;
  // This lane's slot within an item, and its words of `ahead`; recomputed at
  // each use (the loop body needs every register).
  auto lane_slot = [&] { return 32 * S.wave + (fresh(S.lane) & 31); };
  auto ahead_at = [&](int k) -> int & { return ahead[k][64 * S.wave + fresh(S.lane)]; };
  const unsigned ntok_lds = lds_addr(&ahead[1][64 * S.wave]);
  const unsigned nent_lds = lds_addr(&ahead[2][64 * S.wave]);
  auto uni = [](unsigned x) { return (unsigned)__builtin_amdgcn_readfirstlane(x); };
  constexpr unsigned QB = sizeof(Qs[0]), GB = sizeof(Gs[0]), SB = sizeof(st[0]),
                     RB = sizeof(rib[0][0]);

  PagedUnits W;
  {
    const int U = p.items * p.kv_heads, x = blockIdx.x & 7;
    W.per = gridDim.x >> 3;  // the grid is a multiple of 8
    W.j = blockIdx.x >> 3;
    W.ub = x * (U >> 3) + min(x, U & 7);
    W.cnt = (U >> 3) + (x < (U & 7) ? 1 : 0);
  }
  S.io_q.init(D);
  S.io_g.init(D);

  auto rows_of = [&](const PagedSeg &L) -> LinkRows<T> {
    const int hg = L.g * p.group;
    return LinkRows<T>{(const T *)p.q + (int64_t)hg * D, nullptr, (const T *)p.dy + (int64_t)hg * D,
                       p.stats + 3 * (int64_t)hg, plan + p.off_qh_rh + L.qh0,
                       plan + p.off_qh_pos + L.qh0, L.nqh};
  };
  auto make_current = [&](const LinkRows<T> &L) {
    S.qbase = L.qbase;
    S.gbase = L.gbase;
    S.sbase = L.sbase;
    S.rh_tab = L.rh_tab;
    S.pos_tab = L.pos_tab;
    S.nqh = L.nqh;
    S.c_last = (L.nqh - 1) / ROWS;
  };
  // Rowinfo of chunk j of link L into its slot of bank `bank`; data of chunk j
  // (rowinfo landed) into buffer b.
  auto issue_rows = [&](const LinkRows<T> &L, int j, int bank) {
    issue_rows_at(S, L.rh_tab, L.nqh, j, uni(lds_addr(rib[bank][0]) + (j & 3) * RB));
  };
  auto issue_data = [&](const LinkRows<T> &L, int j, int bank, int b) {
    issue_chunk_of(p, S, L, j, rib[bank][j & 3], uni(lds_addr(st) + b * SB), &Qs[b], &Gs[b],
                   uni(lds_addr(Qs) + b * QB), uni(lds_addr(Gs) + b * GB));
  };
  // The next link: found, its token and (for a new unit) slot entries fetched
  // into `ahead`, its rowinfo of chunks 0 .. 3 into bank `bank`.
  auto look_ahead = [&](const PagedSeg &cur, int bank, PagedSeg &nx, LinkRows<T> &lnx) {
    nx = find_seg(p, S, W, cur.k, cur.li + 1);
    if (nx.k < 0) return;
    lnx = rows_of(nx);
    dma_lds4_at(ntok_lds, plan + p.off_link_tok + nx.li * plan::kItemSlots + lane_slot());
    if (nx.k != cur.k)
      dma_lds4_at(nent_lds, plan + p.off_item_slots + nx.item * plan::kItemSlots + lane_slot());
#pragma unroll
    for (int j = 0; j < 4; ++j) issue_rows(lnx, j, bank);
  };

  PagedSeg C = find_seg(p, S, W, 0, -1);
  if (C.k < 0) return;  // every unit was empty (its zero stores are out)
  {
    const int ent = plan[p.off_item_slots + C.item * plan::kItemSlots + lane_slot()];
    ahead_at(0) = ent;
    load_kv(p, S, ent, C.g);
  }
  zero_acc(S);
  S.tok = plan[p.off_link_tok + C.li * plan::kItemSlots + lane_slot()];
  LinkRows<T> LC = rows_of(C), LN;
  make_current(LC);
  int bank = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) issue_rows(LC, j, 0);
  wait_vmem();
  issue_data(LC, 0, 0, 0);
  if (S.c_last >= 1) issue_data(LC, 1, 0, 1);
  S.buf = 0;
  PagedSeg N;
  look_ahead(C, 1, N, LN);
  wait_vmem();
  __syncthreads();

  for (;;) {
    const bool has_next = N.k >= 0, next_unit = has_next && N.k != C.k;
    const int c_last = S.c_last, n_clast = has_next ? (N.nqh - 1) / ROWS : -1;
    // Step c: consume chunk c, then request position c + 2 of the chunk
    // stream (this link's chunk c + 2 with its rowinfo c + 4, else the next
    // link's chunk c + 1 - c_last, whose rowinfo came with the look-ahead) and
    // wait for position c + 1 only (`after` counts the loads issued after it).
    // The loads go out after the body: issued before it, their landing in LDS
    // slows the body's operand reads.
    auto step = [&](auto masked_c, int c) {
      constexpr bool MASKED = decltype(masked_c)::value;
      const int bc = S.buf, b1 = bc == 2 ? 0 : bc + 1, b2 = bc == 0 ? 2 : bc - 1;
      consume_chunk<MASKED>(p, S, c, st[bc], &Qs[bc], &Gs[bc]);
      int after = 0;
      if (c + 2 <= c_last) {
        issue_rows(LC, c + 4, bank);  // its slot's rowinfo (chunk c) was used at step c - 2
        issue_data(LC, c + 2, bank, b2);
        after = PC;
      } else if (has_next) {
        const int j = c + 1 - c_last;
        if (j == 1 && c_last == 0) {  // the next link's chunk 0 is position c + 1: not yet out
          issue_data(LN, 0, bank ^ 1, b1);
          if (n_clast >= 1) {
            issue_data(LN, 1, bank ^ 1, b2);
            after = PD;
          }
        } else if (j <= n_clast) {
          issue_data(LN, j, bank ^ 1, b2);
          after = PD;
        }
      }
      wait_vmem_upto<PD, PC>(after);
      __syncthreads();
      S.buf = b1;
    };
    if (C.masked) {
      for (int c = 0; c <= c_last; ++c) step(std::true_type(), c);
    } else {
      for (int c = 0; c <= c_last; ++c) step(std::false_type(), c);
    }
    if (!has_next) break;
    if (next_unit) {
      // Unit switch (the last step ended with a barrier): the next unit's K / V
      // loads go out first, then the finished unit's rows are staged in its
      // last chunk's buffer and stored.
      const int nent = ahead_at(2);
      load_kv(p, S, nent, N.g);
      const int sb = S.buf == 0 ? 2 : S.buf - 1;  // (S.buf + 2) % 3: the last chunk's buffer
      char *stage = (S.wave < 2 ? reinterpret_cast<char *>(&Qs[sb]) : reinterpret_cast<char *>(&Gs[sb])) +
                    (S.wave & 1) * RowStore<T, D>::BYTES;
      store_unit_rows_seq(p, S, ahead_at(0), &ahead[0][64 * S.wave], C.g, stage);
      ahead_at(0) = nent;
      zero_acc(S);
      __syncthreads();  // staged rows read before the next link's step 0 refills that buffer
    }
    S.tok = ahead_at(1);
    C = N;
    LC = LN;
    make_current(LC);
    bank ^= 1;
    look_ahead(C, bank ^ 1, N, LN);
    // With fewer than three chunks, the steps request the link after next's
    // first chunks (and the last one reads its slot entries) before step 0's
    // wait would cover the look-ahead's loads: wait for them here.
    if (S.c_last <= 1 && N.k >= 0) wait_vmem();
  }
  const int sb = S.buf == 0 ? 2 : S.buf - 1;
  char *stage = (S.wave < 2 ? reinterpret_cast<char *>(&Qs[sb]) : reinterpret_cast<char *>(&Gs[sb])) +
                (S.wave & 1) * RowStore<T, D>::BYTES;
  store_unit_rows_seq(p, S, ahead_at(0), &ahead[0][64 * S.wave], C.g, stage);
}

template <typename T, int D, int P, bool MLA>
static hipError_t launch_t(const PagedParams &p, int nblocks, hipStream_t stream) {
  hipLaunchKernelGGL((k_paged_kv_bwd<T, D, P, MLA>), dim3(nblocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_persist(const PagedParams &p, int nwg, hipStream_t stream) {
  hipLaunchKernelGGL((k_paged_kv_persist<D>), dim3(nwg), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_dtype(int D, const PagedParams &p, int nblocks, hipStream_t stream) {
  if (!p.mla) {
    if (D == 32) return launch_t<T, 32, 0, false>(p, nblocks, stream);
    if (D == 64) return launch_t<T, 64, 0, false>(p, nblocks, stream);
    if (D == 128) return launch_t<T, 128, 0, false>(p, nblocks, stream);
    return hipErrorInvalidValue;
  }
  // latent variant: latent width 64 or 128 (bf16 also 192, 256), position-key
  // width 0, 32 or 64
  if (D == 64 && p.P == 0) return launch_t<T, 64, 0, true>(p, nblocks, stream);
  if (D == 64 && p.P == 32) return launch_t<T, 64, 32, true>(p, nblocks, stream);
  if (D == 64 && p.P == 64) return launch_t<T, 64, 64, true>(p, nblocks, stream);
  if (D == 128 && p.P == 0) return launch_t<T, 128, 0, true>(p, nblocks, stream);
  if (D == 128 && p.P == 32) return launch_t<T, 128, 32, true>(p, nblocks, stream);
  if (D == 128 && p.P == 64) return launch_t<T, 128, 64, true>(p, nblocks, stream);
  if constexpr (sizeof(T) == 2) {  // wider latents: bf16 (32-row chunks)
    if (D == 192 && p.P == 0) return launch_t<T, 192, 0, true>(p, nblocks, stream);
    if (D == 192 && p.P == 32) return launch_t<T, 192, 32, true>(p, nblocks, stream);
    if (D == 192 && p.P == 64) return launch_t<T, 192, 64, true>(p, nblocks, stream);
    if (D == 256 && p.P == 0) return launch_t<T, 256, 0, true>(p, nblocks, stream);
    if (D == 256 && p.P == 32) return launch_t<T, 256, 32, true>(p, nblocks, stream);
    if (D == 256 && p.P == 64) return launch_t<T, 256, 64, true>(p, nblocks, stream);
  }
  return hipErrorInvalidValue;
}

// Compute units of the current device (0 if unknown), looked up once per device.
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0)
      n = 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// nblocks = items * kv_heads units.  workgroups: 0 = pick the form (persistent
// with one workgroup per CU when the units outnumber the CUs); > 0 = the
// persistent form with that many workgroups (a multiple of 8, at least 8; at
// most the unit count rounded up to 8), where it exists (bf16, not latent);
// -1 = one workgroup per unit.
hipError_t launch_paged(bool bf16_in, int D, const PagedParams &p, int nblocks, int workgroups,
                        hipStream_t stream) {
  if (bf16_in && !p.mla) {
    int nwg = 0;
    if (workgroups > 0) {
      nwg = max(8, workgroups / 8 * 8);
    } else if (workgroups == 0) {
      const int cus = device_cus() / 8 * 8;
      if (cus >= 8 && nblocks > cus) nwg = cus;
    }
    if (nwg > 0) {
      nwg = min(nwg, (nblocks + 7) / 8 * 8);
      if (D == 32) return launch_persist<32>(p, nwg, stream);
      if (D == 64) return launch_persist<64>(p, nwg, stream);
      if (D == 128) return launch_persist<128>(p, nwg, stream);
      return hipErrorInvalidValue;
    }
  }
  return bf16_in ? launch_dtype<bf16>(D, p, nblocks, stream)
                 : launch_dtype<float>(D, p, nblocks, stream);
}

}  // namespace attn
