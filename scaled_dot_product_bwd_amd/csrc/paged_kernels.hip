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
template <typename T_, int D_, int P_, bool MLA_> struct PagedState {
  typedef T_ T;
  typedef MT<T> M;
  static constexpr int D = D_, P = P_, DK = D_ + P_;
  static constexpr bool MLA = MLA_;
  static constexpr int NSD = DK / M::KS, NSV = D / M::KS, NT = DK / 32, NTV = D / 32;
  static constexpr int ROWS = KvShape<T>::ROWS;
  typedef Tile<T, DK, ROWS> QTile;  // Q rows (latent variant: [q | qp])
  typedef Tile<T, D, ROWS> GTile;   // dY rows
  typename M::frag kf[NSD], vf[MLA ? 1 : NSV];
  f32x16 dk[NT], dv[MLA ? 1 : NTV];  // latent variant: dk holds both derivatives
  ChunkIO<T, DK, ROWS> io_q;
  ChunkIO<T, D, ROWS> io_g;
  const T *qbase, *qpbase, *gbase;  // Q / qp / dY at head g * group
  const float *sbase;               // statistics at head g * group
  const int32_t *rh_tab, *pos_tab;  // the link's sequence: qh rows from 0
  int nqh, c_last, tok, maxtok, wave, lane, buf;
};

// Rowinfo of chunk c into this wave's copy: lane l <- rh of qh row c * ROWS + l
// (clamped to the last row, so every lane reads inside the plan).
template <typename St>
__device__ __forceinline__ void issue_rowinfo(St &S, int c, int *ri) {
  issue_rowinfo_at(S, c, lds_addr(ri));
}
// The same into the buffer at LDS byte address ri_lds (an integer, so a buffer
// picked at run time costs no generic-pointer arithmetic).
template <typename St>
__device__ __forceinline__ void issue_rowinfo_at(St &S, int c, unsigned ri_lds) {
  const int qh = min(c * St::ROWS + S.lane, S.nqh - 1);
  dma_lds4_at(__builtin_amdgcn_readfirstlane(ri_lds + 4u * 64 * S.wave), S.rh_tab + qh);
}

// Statistics and Q / dY rows of chunk c; `ri` holds the chunk's rowinfo (landed).
// With direct-to-LDS loads the buffers are addressed by their LDS byte
// addresses (integers: st_lds, q_lds, g_lds); register-staged loads (fp32) go
// through the tile pointers.
template <typename St>
__device__ __forceinline__ void issue_chunk(const PagedParams &p, St &S, int c, const int *ri,
                                            unsigned st_lds, typename St::QTile *Q,
                                            typename St::GTile *G, unsigned q_lds,
                                            unsigned g_lds) {
  typedef typename St::T T;
  constexpr int D = St::D, P = St::P;
  const int *myri = ri + 64 * S.wave;
  const unsigned myst = __builtin_amdgcn_readfirstlane(st_lds + 4u * kStatWave * S.wave);
  const int rh = myri[S.lane];
  const float *srow = S.sbase + 3 * (int64_t)rh;
  dma_lds4_at(myst, srow);
  dma_lds4_at(myst + 4u * 64, srow + 1);
  dma_lds4_at(myst + 4u * 128, srow + 2);
  dma_lds4_at(myst + 4u * 192, S.pos_tab + min(c * St::ROWS + S.lane, S.nqh - 1));
  auto qelem = [&](int r, int col) {
    if constexpr (P > 0)  // a row of the tile is [q | qp]: columns below D from q, the rest from qp
      return col < D ? S.qbase + (int64_t)myri[r] * D + col
                     : S.qpbase + (int64_t)myri[r] * P + (col - D);
    else
      return S.qbase + (int64_t)myri[r] * D + col;
  };
  auto gelem = [&](int r, int col) { return S.gbase + (int64_t)myri[r] * D + col; };
  if constexpr (ChunkIO<T, St::DK, St::ROWS>::DIRECT) {
    S.io_q.issue_elem_at(qelem, q_lds);
    S.io_g.issue_elem_at(gelem, g_lds);
  } else {
    S.io_q.issue_elem(qelem, *Q);
    S.io_g.issue_elem(gelem, *G);
  }
}
template <typename St>
__device__ __forceinline__ void issue_chunk(const PagedParams &p, St &S, int c, const int *ri,
                                            float *st, typename St::QTile *Q,
                                            typename St::GTile *G) {
  issue_chunk(p, S, c, ri, lds_addr(st), Q, G, lds_addr(Q), lds_addr(G));
}

// Replace max by -lse2 / scale_log2 in this wave's statistics of chunk c
// (landed): the kv body's starting score.  Rows past the sequence's last qh
// row get -inf, so P = 0 for them with or without the per-element test.  The
// latent variant, whose V fragments are not negated, also negates delta.
template <typename St>
__device__ __forceinline__ void convert_stats(const PagedParams &p, St &S, int c, float *st) {
  float *myst = st + kStatWave * S.wave;
  const int l = S.lane;
  const bool real = l < St::ROWS && c * St::ROWS + l < S.nqh;
  const float m = myst[l], den = myst[64 + l];
  myst[l] = ((real && den > 0.f) ? -fmaf(m, kLog2e, log2f(den)) : -INFINITY) * p.inv_scale_log2;
  if constexpr (St::MLA) myst[128 + l] = -myst[128 + l];
}

// One chunk: request rowinfo of chunk c + 4 and the data of chunk c + 2,
// convert and consume chunk c (MASKED: per-element visibility), hand over.
// Chunk k's tiles, statistics and rowinfo sit in buffer k % 3 (S.buf = c % 3).
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
  convert_stats(p, S, c, st[bc]);
  const float *myst = st[bc] + kStatWave * S.wave;
  const int *posv = reinterpret_cast<const int *>(myst + 192);
  const int tok = S.tok, half = S.lane >> 5;
  const bool causal = p.causal;
  // Slot visible to the row: its token exists and, when causal, is <= the position.
  auto adj = [&](int u, int r) -> float {
    const bool vis = tok >= 0 && (!causal || tok <= posv[32 * u + kr(r, half)]);
    return vis ? 0.f : -INFINITY;
  };
  kv_chunk<T, St::DK, St::D, MASKED, St::MLA, !St::MLA>(S.kf, St::MLA ? S.kf : S.vf, S.dk, S.dv, &Qs[bc],
                                              &Gs[bc], myst, myst + 128, p.scale_log2, S.lane,
                                              adj, p.scale);
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

// One link: all chunks of the sequence's qh rows (rowinfo of chunk k fetched at
// step k - 4, read at step k - 2).  The link runs the unmasked body when every
// lane holds a token that every row of the sequence sees; otherwise the masked
// one.  Each variant has its own loop.
template <typename St>
__device__ __forceinline__ void paged_run(const PagedParams &p, St &S, bool masked,
                                          typename St::QTile *Qs, typename St::GTile *Gs,
                                          float (*st)[kStatWords], int (*ri)[kRiWords]) {
  const int c_last = S.c_last;
  issue_rowinfo(S, 0, ri[0]);
  issue_rowinfo(S, 1, ri[1]);
  issue_rowinfo(S, 2, ri[2]);
  wait_vmem();
  issue_chunk(p, S, 0, ri[0], st[0], &Qs[0], &Gs[0]);
  S.io_q.complete(Qs[0]);
  S.io_g.complete(Gs[0]);
  if (c_last >= 1) {
    issue_chunk(p, S, 1, ri[1], st[1], &Qs[1], &Gs[1]);
    S.io_q.complete(Qs[1]);
    S.io_g.complete(Gs[1]);
  }
  issue_rowinfo(S, 3, ri[0]);
  wait_vmem();
  __syncthreads();
  S.buf = 0;
  if (masked) {
    for (int c = 0; c <= c_last; ++c) paged_step<true>(p, S, c, Qs, Gs, st, ri);
  } else {
    for (int c = 0; c <= c_last; ++c) paged_step<false>(p, S, c, Qs, Gs, st, ri);
  }
}

template <typename T, int D, int P, bool MLA>
__global__ __launch_bounds__(256) void k_paged_kv_bwd(const PagedParams p) {
  typedef PagedState<T, D, P, MLA> St;
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = St::NSD, NT = St::NT, NTV = St::NTV;
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
  const T *krow = (const T *)p.k_pool + srow * D;
  const T *kprow = (const T *)p.kp_pool + srow * P;
#pragma unroll
  for (int s = 0; s < NSD; ++s) {
    const int d0 = s * KS + half * KL;
    S.kf[s] = d0 < D ? load_frag<T>(krow, d0, live) : load_frag<T>(kprow, d0 - D, live);
  }
  if constexpr (!MLA) {
    const T *vrow = (const T *)p.v_pool + srow * D;
#pragma unroll
    for (int s = 0; s < St::NSV; ++s)
      S.vf[s] = neg_frag<T>(load_frag<T>(vrow, s * KS + half * KL, live));  // -V
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) S.dk[t] = f32x16{};
#pragma unroll
  for (int t = 0; t < (MLA ? 1 : NTV); ++t) S.dv[t] = f32x16{};
  S.io_q.init(St::DK);
  S.io_g.init(D);
  const int hg = g * p.group;
  S.qbase = (const T *)p.q + (int64_t)hg * D;
  S.qpbase = (const T *)p.qp + (int64_t)hg * P;
  S.gbase = (const T *)p.dy + (int64_t)hg * D;
  S.sbase = p.stats + 3 * (int64_t)hg;

  const int lb = plan[p.off_item_links + item], le = plan[p.off_item_links + item + 1];
  for (int li = lb; li < le; ++li) {
    const int seq = plan[p.off_link_seq + li];
    const int32_t *info = plan + p.off_link_info + plan::LINK_INFO_WORDS * li;
    const int mintok = info[plan::LI_MIN_TOK];
    if (p.causal && mintok > plan[p.off_seq_maxpos + seq]) continue;  // no row sees the item
    const int qh0 = plan[p.off_seq_qh + seq];
    S.nqh = plan[p.off_seq_qh + seq + 1] - qh0;
    if (S.nqh <= 0) continue;
    S.maxtok = info[plan::LI_MAX_TOK];
    S.tok = plan[p.off_link_tok + li * plan::kItemSlots + 32 * S.wave + l32];
    S.rh_tab = plan + p.off_qh_rh + qh0;
    S.pos_tab = plan + p.off_qh_pos + qh0;
    S.c_last = (S.nqh - 1) / St::ROWS;
    const bool masked = !(info[plan::LI_ALL_VALID] != 0 &&
                          (!p.causal || plan[p.off_seq_minpos + seq] >= S.maxtok));
    paged_run(p, S, masked, Qs, Gs, st, ri);
  }

  // One store per (slot, KV head) element: the gradient, +0 for a tail slot;
  // unused lanes (no slot) store nothing.  Whole rows through LDS when the
  // staging fits the chunk tiles (free once every wave is done).
  const float sc = live ? p.scale : 0.f;  // dS's factor, applied once; tails store +0
  typedef RowStore<T, D> RSd;
  typedef RowStore<T, (P > 0 ? P : 32)> RSp;
  if constexpr (4 * (RSd::BYTES + (MLA && P > 0 ? RSp::BYTES : 0)) <= sizeof(Qs) &&
                4 * RSd::BYTES <= sizeof(Gs)) {
    __syncthreads();
    char *l0 = reinterpret_cast<char *>(Qs) + S.wave * RSd::BYTES;
    char *lp = reinterpret_cast<char *>(Qs) + 4 * RSd::BYTES + S.wave * RSp::BYTES;
    char *l1 = reinterpret_cast<char *>(Gs) + S.wave * RSd::BYTES;
    const int32_t *slot_ent = plan + p.off_item_slots + item * plan::kItemSlots + 32 * S.wave;
    auto row_of = [&](int n) -> int64_t {  // pool row of the wave's lane n, -1 for no slot
      const int e = slot_ent[n];
      return e < 0 ? -1 : (int64_t)(e >> 1) * p.kv_heads + g;
    };
    if constexpr (MLA) {
      // dk holds both derivatives already scaled: the latent's tiles, then the position key's
      if (p.need_dk) RSd::write_tiles(S.dk, live ? 1.f : 0.f, l0, S.lane);
      if (P > 0 && p.need_dkp)
        RSp::write_tiles(S.dk + D / 32, live ? 1.f : 0.f, lp, S.lane);
      if (p.need_dk)
        RSd::store_rows(l0, 32, [&](int n) -> T * {
          const int64_t r = row_of(n);
          return r < 0 ? nullptr : (T *)p.dk_pool + r * D;
        }, S.lane);
      if (P > 0 && p.need_dkp)
        RSp::store_rows(lp, 32, [&](int n) -> T * {
          const int64_t r = row_of(n);
          return r < 0 ? nullptr : (T *)p.dkp_pool + r * P;
        }, S.lane);
    } else {
      if (p.need_dk) RSd::write_tiles(S.dk, sc, l0, S.lane);
      if (p.need_dv) RSd::write_tiles(S.dv, live ? 1.f : 0.f, l1, S.lane);
      if (p.need_dk)
        RSd::store_rows(l0, 32, [&](int n) -> T * {
          const int64_t r = row_of(n);
          return r < 0 ? nullptr : (T *)p.dk_pool + r * D;
        }, S.lane);
      if (p.need_dv)
        RSd::store_rows(l1, 32, [&](int n) -> T * {
          const int64_t r = row_of(n);
          return r < 0 ? nullptr : (T *)p.dv_pool + r * D;
        }, S.lane);
    }
    return;
  }
  if (ent < 0) return;
  if constexpr (MLA) {
    // dS was scaled before its products: dk holds the latent's gradient (both
    // derivatives) and then the position key's; tails store +0
    T *dcrow = (T *)p.dk_pool + srow * D;
    T *dprow = (T *)p.dkp_pool + srow * P;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d0 = 32 * t + 8 * q + 4 * half;
        const f32x16 &a = S.dk[t];
        T *dst = t < NTV ? (p.need_dk ? dcrow + d0 : nullptr) : (p.need_dkp ? dprow + (d0 - D) : nullptr);
        if (dst)
          store4<T>(dst, live ? a[4 * q] : 0.f, live ? a[4 * q + 1] : 0.f,
                    live ? a[4 * q + 2] : 0.f, live ? a[4 * q + 3] : 0.f);
      }
  } else {
    T *dkrow = (T *)p.dk_pool + srow * D;
    T *dvrow = (T *)p.dv_pool + srow * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
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

template <typename T, int D, int P, bool MLA>
static hipError_t launch_t(const PagedParams &p, int nblocks, hipStream_t stream) {
  hipLaunchKernelGGL((k_paged_kv_bwd<T, D, P, MLA>), dim3(nblocks), dim3(256), 0, stream, p);
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
  // latent variant: latent width 64 or 128, position-key width 0, 32 or 64
  if (D == 64 && p.P == 0) return launch_t<T, 64, 0, true>(p, nblocks, stream);
  if (D == 64 && p.P == 32) return launch_t<T, 64, 32, true>(p, nblocks, stream);
  if (D == 64 && p.P == 64) return launch_t<T, 64, 64, true>(p, nblocks, stream);
  if (D == 128 && p.P == 0) return launch_t<T, 128, 0, true>(p, nblocks, stream);
  if (D == 128 && p.P == 32) return launch_t<T, 128, 32, true>(p, nblocks, stream);
  if (D == 128 && p.P == 64) return launch_t<T, 128, 64, true>(p, nblocks, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_paged(bool bf16_in, int D, const PagedParams &p, int nblocks,
                        hipStream_t stream) {
  return bf16_in ? launch_dtype<bf16>(D, p, nblocks, stream)
                 : launch_dtype<float>(D, p, nblocks, stream);
}

}  // namespace attn
