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

namespace attn {

enum { PQ_STATS = 0, PQ_DQ = 1 };

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

template <typename T, int D>
static hipError_t launch_t(int stage, const PagedParams &p, int nblocks, hipStream_t stream) {
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
