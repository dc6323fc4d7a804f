// paged_q_kernels.hip -- the query side of the paged, grouped-query backward:
// per (query row, head) the statistics (max, denominator, delta) that ruDNN
// 0.1.43 src/paged_attention/ordered_kernel.rs `history_backward` takes as an
// input (a query-side kernel there produces them per row), and dQ.
//
// One workgroup per (block of 128 qh rows of one sequence, KV head g); a qh row
// is a (query row, head of g's group) pair, as in the paged dK / dV kernel.
// Wave w owns 32 qh rows (one per lane column); their Q and dY rows sit in
// registers.  The sequence's tokens stream through LDS 32 at a time: token t's
// K / V rows are pool slot tok_slot[t] (plan table), fetched by direct-to-LDS
// loads whose slot ids were themselves loaded into LDS two chunks earlier.
// Per chunk, phase A forms S^T = K Q^T and dP^T = V dY^T (q_core.hpp); then
//   statistics: online max m, l = sum 2^(s - m), delta' = sum 2^(s - m) dP,
//               stored as (m ln 2, l, delta' / l);
//   dQ:         P = 2^(s - lse2), dS' = P (dP - delta), dQ^T += K^T dS'^T,
//               stored times `scale`.
// A token is visible to a row iff it lies inside the sequence and, when
// causal, at or before the row's position.  Rows with no visible token get
// (-inf, 0, 0) and a zero dQ row (a zero denominator, which the pages skip).
//
// Split form: the time of the one-workgroup-per-block form is set by the
// longest sequence.  The split form runs one workgroup per (piece of at most
// kQPieceTokens tokens of a block, KV head), longest pieces first, each writing
// its partial statistics (log2-domain max, l, delta') or unscaled partial dQ to
// a workspace; a merge kernel then combines a block's pieces in token order
// (the statistics by rescaling to the common max, dQ by summing) and writes
// the same outputs.
#include "device_common.hpp"
#include "paged.hpp"
#include "q_core.hpp"
#include "sd_core.hpp"

namespace attn {

enum { PQ_STATS = 0, PQ_DQ = 1, PQ_SDQ = 2 };

constexpr int kPqRi = 4 * 64;  // rowinfo words per buffer: one 64-entry copy per wave

template <typename T, int D, int STAGE> struct PqState {
  typedef MT<T> M;
  static constexpr int NSD = D / M::KS, NT = D / 32;
  typename M::frag qf[1][NSD], gf[1][NSD];
  f32x16 dq[NT];               // dQ stage
  float m, l, dl;              // statistics stage
  float nlse, del;             // dQ stage
  int pos, len, c_last, wave, lane, buf;
  bool valid;
  const int32_t *slots;        // the sequence's token -> slot table
  const T *kbase, *vbase;      // pools at KV head g
  ChunkIO<T, D> io_k, io_v;
};

// Slot ids of chunk c's tokens into this wave's rowinfo copy (clamped to the
// last token, so every lane reads inside the table).
template <typename T, int D, int STAGE>
__device__ __forceinline__ void pq_rowinfo(PqState<T, D, STAGE> &S, int c, int *ri) {
  const int t = min(c * 32 + (S.lane & 31), S.len - 1);
  dma_lds4(ri + 64 * S.wave, S.slots + t);
}

template <typename T, int D, int STAGE>
__device__ __forceinline__ void pq_chunk(const PagedParams &p, PqState<T, D, STAGE> &S,
                                         const int *ri, Tile<T, D> *K, Tile<T, D> *V) {
  const int *myri = ri + 64 * S.wave;
  const int64_t rs = (int64_t)p.kv_heads * D;
  S.io_k.issue_at([&](int r) { return S.kbase + myri[r] * rs; }, *K);
  S.io_v.issue_at([&](int r) { return S.vbase + myri[r] * rs; }, *V);
}

template <typename T, int D, int STAGE>
__device__ __forceinline__ void pq_step(const PagedParams &p, PqState<T, D, STAGE> &S, int c,
                                        Tile<T, D> *Ks, Tile<T, D> *Vs, int (*ri)[kPqRi],
                                        bool masked) {
  typedef MT<T> M;
  constexpr int NT = D / 32, CS = M::CSTEPS;
  constexpr int PER_CHUNK = 1 + 2 * ChunkIO<T, D>::LOADS;
  static_assert(PER_CHUNK < 16, "vmcnt budget");
  const int bc = S.buf, bn = bc == 0 ? 2 : bc - 1, bz = bc == 2 ? 0 : bc + 1;
  const bool issued = c + 2 <= S.c_last;
  if (issued) {
    pq_rowinfo(S, c + 4, ri[bz]);  // always with the chunk: a fixed count per step
    pq_chunk(p, S, ri[bn], &Ks[bn], &Vs[bn]);
  }
  f32x16 sacc[1], pacc[1];
  q_phase_a<T, D, 1>(&Ks[bc], &Vs[bc], S.qf, S.gf, sacc, pacc, S.lane);
  const int half = S.lane >> 5, t0 = c * 32;
  float s2[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) s2[r] = sacc[0][r] * p.scale_log2;
  if (masked) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + kr(r, half);
      const bool vis = t < S.len && (!p.causal || t <= S.pos);
      s2[r] = vis ? s2[r] : -INFINITY;
    }
  }
  if constexpr (STAGE == PQ_STATS) {
    float mx = s2[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s2[r]);
    mx = halves_max(mx);
    const float mn = fmaxf(S.m, mx);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float al = fast_exp2(S.m - mu);
    float ls = 0.f, ds = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = fast_exp2(s2[r] - mu);
      ls += pr;
      ds = fmaf(pr, pacc[0][r], ds);
    }
    S.l = fmaf(S.l, al, ls);
    S.dl = fmaf(S.dl, al, ds);
    S.m = mn;
  } else {
    float dsv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) dsv[r] = fast_exp2(s2[r] + S.nlse) * (pacc[0][r] - S.del);
    const Tile<T, D> *Kc = &Ks[bc];
#pragma unroll
    for (int st = 0; st < CS; ++st) {
      const typename M::frag sf = creuse<T>(dsv, st);
#pragma unroll
      for (int t = 0; t < NT; ++t) S.dq[t] = M::mma(Kc->tfrag(32 * t, st, S.lane), sf, S.dq[t]);
    }
  }
  if (issued) {
    S.io_k.complete(Ks[bn]);
    S.io_v.complete(Vs[bn]);
  }
  if (ChunkIO<T, D>::DIRECT && issued)
    wait_vmem_le<PER_CHUNK>();
  else
    wait_vmem();
  __syncthreads();
  S.buf = bz;
}

template <typename T, int D, int STAGE, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_paged_q(const PagedParams p) {
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NT = D / 32;
  __shared__ Tile<T, D> Ks[3], Vs[3];
  __shared__ __attribute__((aligned(16))) int ri[3][kPqRi];

  PqState<T, D, STAGE> S;
  S.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  S.lane = threadIdx.x & 63;
  const int l32 = S.lane & 31, half = S.lane >> 5;
  const int32_t *plan = p.plan;
  // Workgroup -> (query block or piece, KV head): consecutive ids share a
  // block, so the group's KV heads of one sequence run side by side.
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int g = L % p.kv_heads;
  int blk = L / p.kv_heads, piece = 0, tb0 = 0, te0 = INT32_MAX;
  if constexpr (SPLIT) {
    piece = plan[p.off_qpiece_order + blk];
    blk = plan[p.off_qpiece + 3 * piece];
    tb0 = plan[p.off_qpiece + 3 * piece + 1];
    te0 = plan[p.off_qpiece + 3 * piece + 2];
  }
  const int seq = plan[p.off_qblk + 2 * blk], qh_begin = plan[p.off_qblk + 2 * blk + 1];
  const int qs0 = plan[p.off_seq_qh + seq], nqh = plan[p.off_seq_qh + seq + 1] - qs0;
  const int tb = plan[p.off_seq_tok + seq];
  S.len = plan[p.off_seq_tok + seq + 1] - tb;
  S.slots = plan + p.off_tok_slot + tb;

  const int qh = qh_begin + 32 * S.wave + l32;
  S.valid = qh < nqh;
  const int qhc = S.valid ? qh : 0;
  const int64_t rh = (int64_t)plan[p.off_qh_rh + qs0 + qhc] + (int64_t)g * p.group;  // row * heads + head
  S.pos = plan[p.off_qh_pos + qs0 + qhc];
  const T *qrow = (const T *)p.q + rh * D;
  const T *grow = (const T *)p.dy + rh * D;
#pragma unroll
  for (int s = 0; s < NSD; ++s) {
    S.qf[0][s] = load_frag<T>(qrow, s * KS + half * KL, S.valid);
    S.gf[0][s] = load_frag<T>(grow, s * KS + half * KL, S.valid);
  }
  if constexpr (STAGE == PQ_STATS) {
    S.m = -INFINITY;
    S.l = S.dl = 0.f;
  } else {
    const float *st = p.stats + 3 * rh;
    const float m = S.valid ? st[0] : 0.f, den = S.valid ? st[1] : 0.f;
    S.nlse = den > 0.f ? -fmaf(m, kLog2e, log2f(den)) : -INFINITY;
    S.del = S.valid ? st[2] : 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) S.dq[t] = f32x16{};
  }
  S.kbase = (const T *)p.k_pool + (int64_t)g * D;
  S.vbase = (const T *)p.v_pool + (int64_t)g * D;
  S.io_k.init(0);
  S.io_v.init(0);

  // Tokens any row of the sequence can see: [0, min(len, maxpos + 1)) when
  // causal; chunks all of whose tokens every row sees need no per-element test.
  // The split form's piece covers tokens [tb0, te0) (tb0 a multiple of 32).
  const int maxpos = plan[p.off_seq_maxpos + seq], minpos = plan[p.off_seq_minpos + seq];
  const int tend = min(p.causal ? min(S.len, maxpos + 1) : S.len, te0);
  const int c0 = tb0 / 32;
  S.c_last = tend > tb0 ? (tend - 1) / 32 : c0 - 1;
  const int tfull = p.causal ? min(S.len, minpos + 1) : S.len;  // tokens [0, tfull) seen by all
  wait_vmem();
  if (S.c_last >= c0) {
    pq_rowinfo(S, c0, ri[0]);
    pq_rowinfo(S, c0 + 1, ri[1]);
    pq_rowinfo(S, c0 + 2, ri[2]);
    wait_vmem();
    pq_chunk(p, S, ri[0], &Ks[0], &Vs[0]);
    S.io_k.complete(Ks[0]);
    S.io_v.complete(Vs[0]);
    if (S.c_last >= c0 + 1) {
      pq_chunk(p, S, ri[1], &Ks[1], &Vs[1]);
      S.io_k.complete(Ks[1]);
      S.io_v.complete(Vs[1]);
    }
    pq_rowinfo(S, c0 + 3, ri[0]);
    wait_vmem();
    __syncthreads();
    S.buf = 0;
    for (int c = c0; c <= S.c_last; ++c)
      pq_step<T, D, STAGE>(p, S, c, Ks, Vs, ri, c * 32 + 32 > tfull);
  }

  if (!S.valid) return;
  if constexpr (SPLIT) {
    // partial results of this piece: row 32 wave + l32 of the block
    const int64_t prow = ((int64_t)piece * p.kv_heads + g) * kQBlockRows + 32 * S.wave + l32;
    if constexpr (STAGE == PQ_STATS) {
      const float l_tot = halves_sum(S.l);
      const float d_tot = halves_sum(S.dl);
      if (half == 0) store4<float>(p.qws + 4 * prow, S.m, l_tot, d_tot, 0.f);
    } else {
      float *w = p.qws + prow * D;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          store4<float>(w + 32 * t + 8 * q + 4 * half, S.dq[t][4 * q], S.dq[t][4 * q + 1],
                        S.dq[t][4 * q + 2], S.dq[t][4 * q + 3]);
    }
    return;
  }
  if constexpr (STAGE == PQ_STATS) {
    const float l_tot = halves_sum(S.l);
    const float d_tot = halves_sum(S.dl);
    if (half == 0) {
      const bool empty = !(l_tot > 0.f);
      float *st = p.stats_out + 3 * rh;
      st[0] = empty ? -INFINITY : S.m * kLn2;
      st[1] = empty ? 0.f : l_tot;
      st[2] = empty ? 0.f : d_tot / l_tot;
    }
  } else {
    T *dqrow = (T *)p.dq + rh * D;
    const float sc = p.scale;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        store4<T>(dqrow + 32 * t + 8 * q + 4 * half, sc * S.dq[t][4 * q], sc * S.dq[t][4 * q + 1],
                  sc * S.dq[t][4 * q + 2], sc * S.dq[t][4 * q + 3]);
  }
}

// Merge of the split form: one thread per (block, KV head, row of the block)
// for the statistics, per 4 columns of such a row for dQ.  A block's pieces
// are combined in token order.
template <typename T, int D, int STAGE>
__global__ __launch_bounds__(256) void k_paged_q_merge(const PagedParams p) {
  constexpr int PER = STAGE == PQ_STATS ? 1 : D / 4;  // threads per row
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tid >= (int64_t)p.qblocks * p.kv_heads * kQBlockRows * PER) return;
  const int dc = (int)(tid % PER);
  int64_t r = tid / PER;
  const int j = (int)(r % kQBlockRows);
  r /= kQBlockRows;
  const int g = (int)(r % p.kv_heads), b = (int)(r / p.kv_heads);
  const int32_t *plan = p.plan;
  const int seq = plan[p.off_qblk + 2 * b], qh = plan[p.off_qblk + 2 * b + 1] + j;
  const int qs0 = plan[p.off_seq_qh + seq];
  if (qh >= plan[p.off_seq_qh + seq + 1] - qs0) return;
  const int64_t rh = (int64_t)plan[p.off_qh_rh + qs0 + qh] + (int64_t)g * p.group;
  const int p0 = plan[p.off_qblk_piece + b], p1 = plan[p.off_qblk_piece + b + 1];
  if constexpr (STAGE == PQ_STATS) {
    float m = -INFINITY, l = 0.f, d = 0.f;
    for (int pc = p0; pc < p1; ++pc) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(
          p.qws + 4 * (((int64_t)pc * p.kv_heads + g) * kQBlockRows + j));
      const float mn = fmaxf(m, v[0]);
      if (mn == -INFINITY) continue;  // nothing seen yet
      const float a = fast_exp2(m - mn), c = fast_exp2(v[0] - mn);
      l = fmaf(l, a, v[1] * c);
      d = fmaf(d, a, v[2] * c);
      m = mn;
    }
    const bool empty = !(l > 0.f);
    float *st = p.stats_out + 3 * rh;
    st[0] = empty ? -INFINITY : m * kLn2;
    st[1] = empty ? 0.f : l;
    st[2] = empty ? 0.f : d / l;
  } else {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int pc = p0; pc < p1; ++pc)
      acc += *reinterpret_cast<const f32x4 *>(
          p.qws + (((int64_t)pc * p.kv_heads + g) * kQBlockRows + j) * D + 4 * dc);
    const float sc = p.scale;
    store4<T>((T *)p.dq + rh * D + 4 * dc, sc * acc[0], sc * acc[1], sc * acc[2], sc * acc[3]);
  }
}


// ---------------------------------------------------------------------------
// Statistics and dQ in one pass (bf16): the fused query-major chunk step of
// sd_core.hpp (A' = sum P~ (dP - dh) K and B = sum P~ K against the running
// statistics, four contractions per visible triple) over the sequence's tokens
// in chunks of 64, gathered through the token -> slot table.  Chunk c + 2's
// K / V rows are requested under chunk c's phase A, from slot ids that a
// one-dword-per-lane load brought into this wave's LDS copy a step earlier.
// Direct form: the statistics and dQ rows are final.  Split form: each piece
// writes, per row, its partial (mref, mtrue, l, delta', dh) and A', B
// (log2-domain reference mref, unscaled) to the workspace; the merge combines
// a block's pieces in token order.  Workspace of a (piece, KV head) unit,
// planar so that a wave's rows are contiguous: 128 rows x kSdqRec floats of
// statistics, then 128 rows of A' (D floats each), then 128 rows of B.

constexpr int kSdqRec = 8;  // workspace floats of a row's partial statistics

template <int D> struct PsdState {
  typedef MT<bf16> M;
  static constexpr int NSD = D / M::KS, NT = D / 32;
  typename M::frag qf[NSD], gf[NSD];
  f32x16 acc_a[NT], acc_b[NT];
  RowStat st;
  float dh;
  int lane, half, wave;
  int len, hi, c_last;  // hi: the last token the row sees (-1: none)
  const int32_t *slots;
  const bf16 *kbase, *vbase;
  int64_t rs;  // elements between consecutive pool slots
  ChunkIO<bf16, D, kSdKeys> io;  // (the lane's row and column of each load)
};

// Slot ids of chunk x's tokens (clamped to the sequence's last token) into
// this wave's copy in buffer x & 1.
template <int D>
__device__ __forceinline__ void psd_rowinfo(PsdState<D> &S, int x, int (*ri)[kPqRi]) {
  const int t = min(min(x, S.c_last) * kSdKeys + S.lane, S.len - 1);
  dma_lds4(ri[x & 1] + 64 * S.wave, S.slots + t);
}

// Load j (K for j < L, V after) of chunk x into the tiles at LDS addresses
// klds / vlds; sl[j]: the slot of the lane's row of load j.
template <int D>
__device__ __forceinline__ void psd_load(const PsdState<D> &S, int j, const int *sl, unsigned klds,
                                         unsigned vlds) {
  constexpr int L = ChunkIO<bf16, D, kSdKeys>::LOADS;
  const int jj = j < L ? j : j - L;
  int row, col;
  S.io.slot_rc(jj, row, col);
  const bf16 *src = (j < L ? S.kbase : S.vbase) + (int64_t)sl[jj] * S.rs + col;
  dma_lds16_m0((j < L ? klds : vlds) + ((S.wave + 4 * jj) << 10), src);
}

template <int D>
__device__ __forceinline__ void psd_slots(const PsdState<D> &S, int x, const int (*ri)[kPqRi],
                                          int *sl) {
  constexpr int L = ChunkIO<bf16, D, kSdKeys>::LOADS;
  const int *mine = ri[x & 1] + 64 * S.wave;
#pragma unroll
  for (int j = 0; j < L; ++j) {
    int row, col;
    S.io.slot_rc(j, row, col);
    sl[j] = mine[row];
  }
}

// Chunk c (tokens 64 c ..), its K tile in buffer bk of four and its V tile in
// buffer bv of three; chunk c + 2 into K buffer bk + 2 (chunk c - 2's, whose
// phase C ran in step c - 1) and the V buffer chunk c - 1 used (past c_last
// the last chunk again), slot ids of chunk c + 3.  With PREV, chunk c - 1's
// middle and phase C run here too (its K tile in buffer bk - 1).
template <int D, bool MASKED, bool PREV>
__device__ __forceinline__ void psd_step(const PagedParams &p, PsdState<D> &S, int c, int bk, int bv,
                                         Tile<bf16, D, kSdKeys> *Ks, Tile<bf16, D, kSdKeys> *Vs,
                                         int (*ri)[kPqRi], SdCarry<bf16> &X) {
  constexpr int L = ChunkIO<bf16, D, kSdKeys>::LOADS;
  const int kn = (bk + 2) & 3, vn = bv == 0 ? 2 : bv - 1;
  psd_rowinfo(S, c + 3, ri);
  int sl[L];
  psd_slots(S, c + 2, ri, sl);
  constexpr unsigned TB = sizeof(Tile<bf16, D, kSdKeys>);
  const unsigned klds = lds_addr(Ks) + kn * TB, vlds = lds_addr(Vs) + vn * TB;
  auto dma = [&](int k) { psd_load(S, k, sl, klds, vlds); };
  const int half = S.half, t0 = c * kSdKeys;
  auto adj_of = [&](int u, int r) {
    return t0 + 32 * u + kr(r, half) > S.hi ? -INFINITY : 0.f;
  };
  sd_body_deferred<bf16, D, MASKED, PREV>(S, p.scale_log2, &Ks[bk], &Vs[bv], &Ks[(bk + 3) & 3], X,
                                          adj_of, dma);
}

template <int D, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_paged_sdq(const PagedParams p) {
  typedef bf16 T;
  typedef MT<T> M;
  constexpr int KS = M::KS, KL = M::KL, NSD = D / KS, NT = D / 32, KC = kSdKeys;
  __shared__ Tile<T, D, KC> Ks[4], Vs[3];
  __shared__ __attribute__((aligned(16))) int ri[2][kPqRi];

  PsdState<D> S;
  S.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  S.lane = threadIdx.x & 63;
  S.half = S.lane >> 5;
  const int l32 = S.lane & 31, half = S.half;
  const int32_t *plan = p.plan;
  const int L0 = xcd_remap(blockIdx.x, gridDim.x);
  const int g = L0 % p.kv_heads;
  int blk = L0 / p.kv_heads, piece = 0, tb0 = 0, te0 = INT32_MAX;
  if constexpr (SPLIT) {
    piece = plan[p.off_qpiece_order + blk];
    blk = plan[p.off_qpiece + 3 * piece];
    tb0 = plan[p.off_qpiece + 3 * piece + 1];
    te0 = plan[p.off_qpiece + 3 * piece + 2];
  }
  const int seq = plan[p.off_qblk + 2 * blk], qh_begin = plan[p.off_qblk + 2 * blk + 1];
  const int qs0 = plan[p.off_seq_qh + seq], nqh = plan[p.off_seq_qh + seq + 1] - qs0;
  const int tb = plan[p.off_seq_tok + seq];
  S.len = plan[p.off_seq_tok + seq + 1] - tb;
  S.slots = plan + p.off_tok_slot + tb;

  const int qh = qh_begin + 32 * S.wave + l32;
  const bool valid = qh < nqh;
  const int qhc = valid ? qh : 0;
  const int64_t rh = (int64_t)plan[p.off_qh_rh + qs0 + qhc] + (int64_t)g * p.group;
  const int pos = plan[p.off_qh_pos + qs0 + qhc];
  S.hi = !valid ? -1 : p.causal ? min(S.len - 1, pos) : S.len - 1;
  const T *qrow = (const T *)p.q + rh * D;
  const T *grow = (const T *)p.dy + rh * D;
#pragma unroll
  for (int s = 0; s < NSD; ++s) {
    S.qf[s] = load_frag<T>(qrow, s * KS + half * KL, valid);
    S.gf[s] = load_frag<T>(grow, s * KS + half * KL, valid);
  }
  sd_init<NT>(S);
  S.rs = (int64_t)p.kv_heads * D;
  S.kbase = (const T *)p.k_pool + (int64_t)g * D;
  S.vbase = (const T *)p.v_pool + (int64_t)g * D;
  S.io.init(0);

  // Tokens [tb0, tend) in chunks c0 .. c_last; chunks below tfull (seen by
  // every row of the sequence) take the unmasked step when scale > 0.
  const int maxpos = plan[p.off_seq_maxpos + seq], minpos = plan[p.off_seq_minpos + seq];
  const int tend = min(p.causal ? min(S.len, maxpos + 1) : S.len, te0);
  const int c0 = tb0 / KC;
  S.c_last = tend > tb0 ? (tend - 1) / KC : c0 - 1;
  const int tfull = p.causal ? min(S.len, minpos + 1) : S.len;
  wait_vmem();
  if (S.c_last >= c0) {
    int sl[ChunkIO<T, D, KC>::LOADS];
    constexpr int L2 = 2 * ChunkIO<T, D, KC>::LOADS;
    constexpr unsigned TB = sizeof(Tile<T, D, KC>);
    psd_rowinfo(S, c0, ri);
    psd_rowinfo(S, c0 + 1, ri);
    wait_vmem();
    psd_slots(S, c0, ri, sl);
#pragma unroll
    for (int k = 0; k < L2; ++k) psd_load(S, k, sl, lds_addr(Ks), lds_addr(Vs));
    psd_slots(S, c0 + 1, ri, sl);
#pragma unroll
    for (int k = 0; k < L2; ++k) psd_load(S, k, sl, lds_addr(Ks) + TB, lds_addr(Vs) + TB);
    psd_rowinfo(S, c0 + 2, ri);  // into buffer c0 & 1, whose ids were read above
    wait_vmem();
    __syncthreads();
    int cu = min(tfull / KC, S.c_last + 1);  // chunks [c0, cu) unmasked
    if (!(p.scale_log2 > 0.f)) cu = c0;
    int c = c0, bk = 0, bv = 0;
    auto next = [&]() {
      ++c;
      bk = (bk + 1) & 3;
      bv = bv == 2 ? 0 : bv + 1;
    };
    SdCarry<T> X;
    if (c < cu)  // the first chunk has no pending one
      psd_step<D, false, false>(p, S, c, bk, bv, Ks, Vs, ri, X);
    else
      psd_step<D, true, false>(p, S, c, bk, bv, Ks, Vs, ri, X);
    next();
    for (; c < cu; next()) psd_step<D, false, true>(p, S, c, bk, bv, Ks, Vs, ri, X);
    for (; c <= S.c_last; next()) psd_step<D, true, true>(p, S, c, bk, bv, Ks, Vs, ri, X);
    sd_finish<T, D>(S, &Ks[(bk + 3) & 3], X);  // the last chunk's phase C
    wait_vmem();  // the repeated loads of the last steps land before the workgroup ends
  }

  if constexpr (SPLIT) {
    // Partial results of rows 32 wave .. 32 wave + 31 of the unit (an invalid
    // row's are never read).  A' and B go out as whole rows through LDS: the
    // chunk tiles are free once every wave's repeated loads have landed.
    float *u = p.qws + ((int64_t)piece * p.kv_heads + g) * kQBlockRows * (kSdqRec + 2 * D);
    const int r0 = 32 * S.wave;
    const float l_tot = halves_sum(S.st.l);
    const float d_tot = halves_sum(S.st.dl);
    if (half == 0) {
      float *w = u + (r0 + l32) * kSdqRec;
      store4<float>(w, S.st.mref, S.st.mtrue, l_tot, d_tot);
      store4<float>(w + 4, S.dh, 0.f, 0.f, 0.f);
    }
    typedef RowStore<float, D> RS;
    static_assert(2 * RS::BYTES <= sizeof(Ks) && 2 * RS::BYTES <= sizeof(Vs), "staging fits");
    __syncthreads();
    char *area = reinterpret_cast<char *>(S.wave < 2 ? (void *)Ks : (void *)Vs) + (S.wave & 1) * RS::BYTES;
    float *wa = u + kQBlockRows * kSdqRec + (int64_t)r0 * D;
    float *wb = wa + kQBlockRows * D;
    RS::write_tiles(S.acc_a, 1.f, area, S.lane);
    RS::store_rows(area, 32, [&](int n) { return wa + n * D; }, S.lane);
    RS::write_tiles(S.acc_b, 1.f, area, S.lane);  // LDS operations of a wave complete in order
    RS::store_rows(area, 32, [&](int n) { return wb + n * D; }, S.lane);
    return;
  }
  if (!valid) return;
  const RowStatOut o = row_stat_final(S.st, p.inv_scale_log2);
  if (half == 0) {
    float *st = p.stats_out + 3 * rh;
    st[0] = o.m;
    st[1] = o.l;
    st[2] = o.delta;
  }
  sd_settle<NT>(S, o.delta);
  T *dqrow = (T *)p.dq + rh * D;
  const float sc = p.scale * o.inv_l;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      store4<T>(dqrow + 32 * t + 8 * q + 4 * half, sc * S.acc_a[t][4 * q],
                sc * S.acc_a[t][4 * q + 1], sc * S.acc_a[t][4 * q + 2], sc * S.acc_a[t][4 * q + 3]);
}

// Merge of the fused split form: one thread per 4 columns of a (block, KV head,
// row of the block).  Pieces in token order: the common reference M (largest
// mref), l = sum 2^(mref_p - M) l_p and delta' likewise, delta = delta' / l,
// dQ = scale / l * sum 2^(mref_p - M) (A'_p + (dh_p - delta) B_p).  The
// statistics (written by each row's first thread) are (mtrue ln 2,
// l 2^(M - mtrue), delta), as the direct form's.
template <int D>
__global__ __launch_bounds__(256) void k_paged_sdq_merge(const PagedParams p) {
  typedef bf16 T;
  constexpr int PER = D / 4, REC = kSdqRec + 2 * D;
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tid >= (int64_t)p.qblocks * p.kv_heads * kQBlockRows * PER) return;
  const int dc = (int)(tid % PER);
  int64_t r = tid / PER;
  const int j = (int)(r % kQBlockRows);
  r /= kQBlockRows;
  const int g = (int)(r % p.kv_heads), b = (int)(r / p.kv_heads);
  const int32_t *plan = p.plan;
  const int seq = plan[p.off_qblk + 2 * b], qh = plan[p.off_qblk + 2 * b + 1] + j;
  const int qs0 = plan[p.off_seq_qh + seq];
  if (qh >= plan[p.off_seq_qh + seq + 1] - qs0) return;
  const int64_t rh = (int64_t)plan[p.off_qh_rh + qs0 + qh] + (int64_t)g * p.group;
  const int p0 = plan[p.off_qblk_piece + b], p1 = plan[p.off_qblk_piece + b + 1];
  auto unit = [&](int pc) { return p.qws + ((int64_t)pc * p.kv_heads + g) * kQBlockRows * REC; };
  auto rec = [&](int pc) { return unit(pc) + j * kSdqRec; };
  float M = -INFINITY, mt = -INFINITY;
  for (int pc = p0; pc < p1; ++pc) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(rec(pc));
    M = fmaxf(M, v[0]);
    mt = fmaxf(mt, v[1]);
  }
  float l = 0.f, dl = 0.f;
  if (M != -INFINITY) {
    for (int pc = p0; pc < p1; ++pc) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(rec(pc));
      const float a = fast_exp2(v[0] - M);  // 0 for a piece that saw nothing
      l = fmaf(v[2], a, l);
      dl = fmaf(v[3], a, dl);
    }
  }
  const bool empty = !(l > 0.f);
  const float delta = empty ? 0.f : dl / l;
  if (dc == 0) {
    float *st = p.stats_out + 3 * rh;
    st[0] = empty ? -INFINITY : mt * kLn2;
    st[1] = empty ? 0.f : l * fast_exp2(M - mt);
    st[2] = delta;
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (!empty) {
    for (int pc = p0; pc < p1; ++pc) {
      const float *w = rec(pc);
      const f32x4 v = *reinterpret_cast<const f32x4 *>(w);
      if (v[0] == -INFINITY) continue;  // nothing seen in this piece
      const float a = fast_exp2(v[0] - M), sh = w[4] - delta;
      const float *ra = unit(pc) + kQBlockRows * kSdqRec + (int64_t)j * D + 4 * dc;
      const f32x4 A = *reinterpret_cast<const f32x4 *>(ra);
      const f32x4 B = *reinterpret_cast<const f32x4 *>(ra + kQBlockRows * D);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(a, fmaf(sh, B[e], A[e]), acc[e]);
    }
  }
  const float sc = empty ? 0.f : p.scale / l;
  store4<T>((T *)p.dq + rh * D + 4 * dc, sc * acc[0], sc * acc[1], sc * acc[2], sc * acc[3]);
}

template <typename T, int D>
static hipError_t launch_t(int stage, const PagedParams &p, int nblocks, hipStream_t stream) {
  if (stage == PQ_SDQ) {
    if constexpr (sizeof(T) == 2) {
      if (!p.qws) {
        hipLaunchKernelGGL((k_paged_sdq<D, false>), dim3(nblocks), dim3(256), 0, stream, p);
        return hipGetLastError();
      }
      const int64_t mthreads = (int64_t)p.qblocks * p.kv_heads * kQBlockRows * (D / 4);
      hipLaunchKernelGGL((k_paged_sdq<D, true>), dim3(p.qpieces * p.kv_heads), dim3(256), 0,
                         stream, p);
      hipLaunchKernelGGL((k_paged_sdq_merge<D>), dim3((int)((mthreads + 255) / 256)), dim3(256), 0,
                         stream, p);
      return hipGetLastError();
    } else {
      // fp32: the statistics, then dQ from them
      const hipError_t e = launch_t<T, D>(PQ_STATS, p, nblocks, stream);
      if (e != hipSuccess) return e;
      PagedParams p2 = p;
      p2.stats = p.stats_out;
      return launch_t<T, D>(PQ_DQ, p2, nblocks, stream);
    }
  }
  if (!p.qws) {
    if (stage == PQ_STATS)
      hipLaunchKernelGGL((k_paged_q<T, D, PQ_STATS, false>), dim3(nblocks), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((k_paged_q<T, D, PQ_DQ, false>), dim3(nblocks), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  // split form: the pieces, then the merge
  const int npiece = p.qpieces * p.kv_heads;
  const int64_t mthreads =
      (int64_t)p.qblocks * p.kv_heads * kQBlockRows * (stage == PQ_STATS ? 1 : D / 4);
  const int mblocks = (int)((mthreads + 255) / 256);
  if (stage == PQ_STATS) {
    hipLaunchKernelGGL((k_paged_q<T, D, PQ_STATS, true>), dim3(npiece), dim3(256), 0, stream, p);
    hipLaunchKernelGGL((k_paged_q_merge<T, D, PQ_STATS>), dim3(mblocks), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((k_paged_q<T, D, PQ_DQ, true>), dim3(npiece), dim3(256), 0, stream, p);
    hipLaunchKernelGGL((k_paged_q_merge<T, D, PQ_DQ>), dim3(mblocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_paged_q(int stage, bool bf16_in, int D, const PagedParams &p, int nblocks,
                          hipStream_t stream) {
  if (bf16_in) {
    if (D == 32) return launch_t<bf16, 32>(stage, p, nblocks, stream);
    if (D == 64) return launch_t<bf16, 64>(stage, p, nblocks, stream);
    if (D == 128) return launch_t<bf16, 128>(stage, p, nblocks, stream);
  } else {
    if (D == 32) return launch_t<float, 32>(stage, p, nblocks, stream);
    if (D == 64) return launch_t<float, 64>(stage, p, nblocks, stream);
    if (D == 128) return launch_t<float, 128>(stage, p, nblocks, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace attn
